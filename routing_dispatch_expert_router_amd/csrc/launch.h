// Internal interface between the C-ABI host code (moe_api.cpp) and the kernel
// files.  Launchers return 0, -2 (unsupported shape) or -4 (launch error).
#pragma once
#include <algorithm>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Status of the launches since the last check: 0, or -4 (MOE_ERR_HIP) after
// writing HIP's reason and the launch name to stderr when the MOE_DEBUG
// environment variable is set.
int launch_status(const char *what);

// Validated, normalised layer shape.
// keep rules as the kernels see them: the public moe_drop values, and the
// experts' own top-C choice of expert-choice routing
enum { DROP_NONE = 0, DROP_CAPACITY = 1, DROP_AFFINITY = 2, DROP_TOPC = 3 };

struct Shape {
  int T, d, H, dh, E, Eh, k, K;  // K = H * k assignments per token (expert choice: k = K = E)
  int n_groups, topk_groups, renorm;
  int drop, C, keep_num, keep_den;
  int expert_choice, sel_gate, seq_len;
  int dff, act, n_shared, latent, residual;
  bool act_f32, router_f32;
  long R_max;                     // upper bound on kept rows
};

// ---------------------------------------------------------------- route
// route_kernel's launch: grid nbx x H blocks of tb tokens (wt token groups of
// mw*16 tokens, each split over wk waves along d_head); L lanes per token in
// the selection (Lg per expert group with group-limited routing), epl experts
// per lane; st: scores from LDS-staged chunks, the waves splitting the experts
struct RouteGeom {
  int nf, nplanes, mw, wt, wk, tb, nbx;
  int L, Lg, epl, st;
};
RouteGeom route_geometry(const Shape &s);
bool route_supported(const Shape &s);
size_t route_ws_bytes(const Shape &s);
// the router's per-block statistics at the start of its workspace: the
// probability sums [nbx][E], then the choice counts [nbx][E] at
// route_hist_offset(s); route_stats_bytes(s) covers both
size_t route_hist_offset(const Shape &s);
size_t route_stats_bytes(const Shape &s);
// hist_out: [nbx][E] per-block choice counts (blocks of route_geometry(s).tb
// tokens), or NULL
int launch_route(const Shape &s, const void *x, const void *w_router, const float *bias, const float *sel_bias,
                 float *logits, int mode, int32_t *topk_idx, float *topk_w, float *aux_loss, float *seq_loss,
                 void *ws, hipStream_t st, int32_t *hist_out = nullptr);
int launch_sel_bias_update(const Shape &s, const int32_t *load, float *sel_bias, float gamma, hipStream_t st);

// ---------------------------------------------------------------- dispatch
// checked mode: the count of invalid topk_idx slots into *status (one block)
int launch_topk_check(const Shape &s, const int32_t *topk_idx, int32_t *status, hipStream_t st);
size_t dispatch_ws_bytes(const Shape &s);
// workspace of a dispatch that takes the router's choice counts (route_hist,
// left in the same workspace at route_hist_offset(s) by launch_route)
size_t dispatch_after_route_ws_bytes(const Shape &s);
// the library-held dispatch scratch (moe_dispatch_noalloc): its size, and
// its device address on the current device (0, or -4 when HIP fails)
constexpr size_t DISPATCH_SCRATCH_MAX = (size_t)8 << 20;
int dispatch_scratch(void **out);
int launch_dispatch(const Shape &s, const int32_t *topk_idx, const float *topk_w, const void *x,
                    int32_t *demand, int32_t *counts, int32_t *offsets, int32_t *row_of, int32_t *src_of,
                    void *x_perm, void *ws, hipStream_t st, const int32_t *route_hist = nullptr);

// ---------------------------------------------------------------- backward
// grouped-GEMM epilogues the backward selects at run time
enum { GEMM_EPI_PLAIN = 0, GEMM_EPI_SWIGLU_BWD = 4, GEMM_EPI_RELU_BWD = 5 };
int gemm_routed(const Shape &s, int epi, const void *A, long lda, const int32_t *gather, const void *B,
                const void *B2, long ldb, long bstride, void *C, long ldc, int N, int K, const int32_t *offsets,
                const void *dh, long lddh, void *hout, long ldh, int32_t *prefix, hipStream_t st);
int gemm_plain(bool f32, int epi, const void *A, long lda, const void *B, const void *B2, long ldb, void *C,
               long ldc, int M, int N, int K, const void *dh, long lddh, void *hout, long ldh, hipStream_t st);
// The K-grouped products below read A [M rows][K] and B [N rows][K] k-chunked
// (launch_transpose with kchunk): (row, k) at (k / KC) * ld * KC + row * KC +
// k % KC, KC = the elements of 128 bytes, lda / ldb = the buffers' row counts.
// one group's C[M, N] = A B^T over K windows kwin[0..nsplit] (multiples of 64),
// through float32 partials part[nsplit][M][N] added in order
int gemm_splitk(bool f32, const void *A, long lda, const void *B, long ldb, void *C, int M, int N, int nsplit,
                const int32_t *kwin, float *part, hipStream_t st);
int splitk_count(bool f32, int M, int N, long K);
// K-grouped products with every group's window cut in pieces of at most
// `depth` columns (kgroup_piece_depth): whole windows write C directly, cut
// ones go through float32 partials (part: kgroup_max_slots x M x N floats)
// added in order.  tab: 4 * max_pieces + 1 ints; red: 2 * G ints.
int kgroup_piece_depth(bool f32, int G, int M, int N, long Rp);
long kgroup_max_pieces(int G, long Rp, int depth);
long kgroup_max_slots(long Rp, int depth);
int gemm_kgrouped_pieces(bool f32, const void *A, long lda, const void *B, long ldb, void *C, long ldc, long cstride,
                         int G, int M, int N, const int32_t *kwin, int depth, long max_pieces, int32_t *tab,
                         int32_t *red, float *part, hipStream_t st);
// fused expert MLP (mlp.hip): bf16, d_e of 64, 128 or 256, d_ff a multiple
// of 32; prefix: E + 1 ints of workspace
bool mlp_fused_supported(const Shape &s);
// The combine of a layer whose every (token, head) holds exactly one kept
// assignment, done by the expert FFN's epilogue: row r's output, times its
// gate w[asg[r]], goes to o[asg[r] / K][h * d_head ..] (h = the row's
// expert's head), rounded as the combine rounds it.  o == NULL: no fold.
struct FoldOut {
  void *o;
  const float *w;
  const int32_t *asg;
};
bool fold_supported(const Shape &s);
int launch_mlp_fused(const Shape &s, const void *xin, const int32_t *gather, const int32_t *offsets, const void *w1,
                     const void *w3, const void *w2, void *y_perm, int32_t *prefix, hipStream_t st,
                     const FoldOut &fold = FoldOut{});
// kchunk: dst k-chunked (ld_dst = its row count, njcols a multiple of 64), else row-major
int launch_transpose(bool f32, const void *src, long ld_src, long bs_src, const int32_t *rmap, long nvalid,
                     long njcols, int ncols, int coff, void *dst, long ld_dst, long bs_dst, int batches,
                     hipStream_t st, int kchunk = 0);
int launch_bwd_rows(const Shape &s, const void *dy, long ld_dy, const void *y_perm, const float *gates,
                    const int32_t *src_of, const int32_t *topk_idx, const int32_t *offsets, void *dY, float *dg,
                    hipStream_t st);
// the backward's activation step from the forward's kept pre-activations gu
// (see launch_expert_ffn): dA|dB [R][m d_ff] and H [R][d_ff] from gu and the
// upstream dH [R][d_ff], for rows below offsets[E]
int launch_bwd_saved_act(const Shape &s, const void *gu, const void *dH, void *dAB, void *H, const int32_t *offsets,
                         hipStream_t st);
int launch_bwd_pad(const Shape &s, const int32_t *offsets, const int32_t *src_of, int32_t *poff, int32_t *pmap_r,
                   int32_t *pmap_x, long npad, hipStream_t st);
// float32 layers: the router weight gradient sums router_wgrad_split(s) token
// ranges separately (enough 64 x 64 tiles to fill the chip), then adds them in
// order
inline int router_wgrad_split(const Shape &s) {
  const long tiles = (long)s.H * ((s.Eh + 63) / 64) * ((s.dh + 63) / 64);
  return (int)std::min<long>(64, std::max<long>(1, (4096 + tiles - 1) / std::max<long>(tiles, 1)));
}
// bf16 layers take the router weight gradient on MFMA: dl as three bf16
// planes (hi + mid + lo = dl to float32 accuracy), transposed per head to
// [H][3][ep][tp] (ep = E_h rounded up to the tile's bm experts, tp = T rounded
// up to 64), against x rows read through transposing LDS reads.  Tiles of bm
// experts x 256 columns; the tokens split in nsplit ranges of `per` (a
// multiple of 64), float32 partials added in order.
struct RouterWgradGeom {
  int bm, ep, tp, per, nsplit;
};
inline RouterWgradGeom router_wgrad_geom(const Shape &s) {
  RouterWgradGeom g;
  g.bm = s.Eh <= 16 ? 16 : s.Eh <= 32 ? 32 : 64;
  g.ep = (s.Eh + g.bm - 1) / g.bm * g.bm;
  g.tp = (int)(((long)s.T + 63) / 64 * 64);
  const long tiles = (long)s.H * (g.ep / g.bm) * ((s.dh + 255) / 256);
  // resident blocks: LDS per block is 2 x (3 bm x 128 + 33792) bytes, so two
  // 16-expert blocks fit a CU's 160 KiB, one of the wider ones
  const long slots = g.bm == 16 ? 512 : 256;
  const long chunks = std::max<long>(1, g.tp / 64);
  const long want = std::min<long>(64, std::max<long>(1, slots / tiles));
  g.per = (int)((chunks + want - 1) / want * 64);
  g.nsplit = (int)std::max<long>(1, ((long)s.T + g.per - 1) / g.per);
  return g;
}
inline size_t router_planes_bytes(const Shape &s) {
  if (s.act_f32) return 0;
  const RouterWgradGeom g = router_wgrad_geom(s);
  return (size_t)s.H * 3 * g.ep * g.tp * 2;
}
// float32 partials of the router weight and bias gradients: the weight
// gradient's token ranges (E x d_head each), and ROUTER_DBIAS_CHUNKS x E for
// the bias gradient (used first, in stream order)
constexpr int ROUTER_DBIAS_CHUNKS = 256;
inline size_t router_part_floats(const Shape &s) {
  const long parts = s.act_f32 ? router_wgrad_split(s) : router_wgrad_geom(s).nsplit;
  return (size_t)std::max<long>(parts * s.dh, ROUTER_DBIAS_CHUNKS) * s.E;
}
// planes: router_planes_bytes(s) of workspace (bf16 layers)
int launch_router_bwd(const Shape &s, const float *logits, const int32_t *topk_idx, const float *gates,
                      const float *dg, const int32_t *demand, float lam, const int32_t *seq_cnt, float seq_w,
                      const void *x, float *dl, uint16_t *planes, float *part, float *dw_router, float *dbias,
                      hipStream_t st);
// seq_cnt[s][e]: choices of expert e within sequence s
int launch_seq_counts(const Shape &s, const int32_t *topk_idx, int32_t *seq_cnt, hipStream_t st);
int launch_bwd_dx(const Shape &s, const void *dy, const void *dxs, const void *dXr, const int32_t *row_of,
                  const float *dl, const void *w_router, int residual, void *dx, hipStream_t st);
// kwin[s] = s * tpad / nsplit rounded up to 64 (kwin[nsplit] = tpad)
int launch_set_kwin(int32_t *kwin, int tpad, int nsplit, hipStream_t st);

// ---------------------------------------------------------------- grouped GEMM / expert FFN
size_t ffn_ws_bytes(const Shape &s);
// gather == NULL: `xin` is x_perm (row r of the routed operand is xin[r]);
// else `xin` is the expert input x and row r is read from x[gather[r] / K]
// at column offset (e / E_h) * d_head
// fold.o != NULL (fold_supported(s) only): the combine folded into the
// epilogue (see FoldOut); y_perm may then be NULL (not written).  gsave !=
// NULL (ffn_grouped(s) only): the routed gate/up products' pre-activations
// are kept there, [R_max][2 d_ff] (SwiGLU: gate, then up) or [R_max][d_ff]
// (ReLU), act dtype, rows as y_perm
int launch_expert_ffn(const Shape &s, const void *xin, const int32_t *gather, const int32_t *offsets,
                      const void *w1, const void *w3, const void *w2, void *y_perm, const void *x_shared,
                      const void *ws1, const void *ws3, const void *ws2, void *shared_out, void *ws, hipStream_t st,
                      const FoldOut &fold = FoldOut{}, void *gsave = nullptr);
// whether the routed experts run the grouped GEMM (not the fused MLP): the
// layers whose forward can keep the pre-activations for the backward
bool ffn_grouped(const Shape &s);
// dense C[M,N] = A[M,K] B[N,K]^T (+ residual R[M,N]), act dtype, float32 accumulate
size_t dense_ws_bytes();
int launch_dense(bool f32, const void *A, const void *B, void *C, const void *residual, int M, int N, int K,
                 void *ws, hipStream_t st);

// ---------------------------------------------------------------- combine
int launch_combine(const Shape &s, const void *y_perm, const int32_t *row_of, const float *topk_w,
                   const void *residual, const void *shared_out, void *y, hipStream_t st);

}  // namespace moe

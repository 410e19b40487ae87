// C-ABI entry points of libmoe.so (declared and documented in include/moe.h).
// Host code only: validation, workspace layout and launch order.  Every check
// runs before the first launch, so a rejected call launches nothing.
#include <initializer_list>
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/moe.h"
#include "launch.h"

using moe::Shape;

int moe::launch_status(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return 0;
  if (getenv("MOE_DEBUG")) fprintf(stderr, "moe: %s launch failed: %s\n", what, hipGetErrorString(e));
  return -4;
}

namespace {

size_t al(size_t v) { return (v + 255) / 256 * 256; }

// config -> Shape; returns a moe_status
int make_shape(const moe_config *c, Shape *s) {
  if (!c) return MOE_ERR_ARG;
  if (c->T < 0 || c->d_model <= 0 || c->d_model % 64 || c->n_heads < 1 || c->d_head <= 0 || c->d_head % 64)
    return MOE_ERR_ARG;
  if (!c->latent_proj && (long)c->n_heads * c->d_head != c->d_model) return MOE_ERR_ARG;
  if (c->n_experts < 1 || c->n_experts % c->n_heads) return MOE_ERR_ARG;
  const int Eh = c->n_experts / c->n_heads;
  const bool ec = c->route_mode == MOE_ROUTE_EXPERT_CHOICE;  // top_k unused: every expert is a slot
  if (!ec && (c->top_k < 1 || c->top_k > Eh)) return MOE_ERR_ARG;
  if (c->n_groups < 0) return MOE_ERR_ARG;
  if (c->n_groups > 0) {
    if (Eh % c->n_groups || c->topk_groups < 1 || c->topk_groups > c->n_groups) return MOE_ERR_ARG;
    if (!ec && (long)c->top_k > (long)c->topk_groups * (Eh / c->n_groups)) return MOE_ERR_ARG;
  }
  if ((c->renorm != 0 && c->renorm != 1) || c->drop < 0 || c->drop > 2) return MOE_ERR_ARG;
  if ((c->route_mode != MOE_ROUTE_TOKEN_CHOICE && c->route_mode != MOE_ROUTE_EXPERT_CHOICE) ||
      (c->sel_bias_gate != 0 && c->sel_bias_gate != 1) || c->seq_len < 0)
    return MOE_ERR_ARG;
  if (c->seq_len > 0 && c->T % c->seq_len) return MOE_ERR_ARG;
  if (ec && (c->drop != MOE_DROP_CAPACITY || c->renorm)) return MOE_ERR_ARG;
  if (c->drop == MOE_DROP_CAPACITY && c->capacity < 0) return MOE_ERR_ARG;
  if (c->drop == MOE_DROP_AFFINITY && (c->keep_num <= 0 || c->keep_den <= 0 || c->keep_num > c->keep_den))
    return MOE_ERR_ARG;
  if (c->d_ff <= 0 || c->d_ff % 64 || (c->act != MOE_ACT_RELU && c->act != MOE_ACT_SWIGLU)) return MOE_ERR_ARG;
  if (c->n_shared < 0 || (c->latent_proj != 0 && c->latent_proj != 1) || (c->residual != 0 && c->residual != 1))
    return MOE_ERR_ARG;
  if ((c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16) ||
      (c->router_dtype != MOE_F32 && c->router_dtype != MOE_BF16))
    return MOE_ERR_ARG;
  // supported subset
  if ((!ec && c->top_k > 8) || Eh > 256 || c->n_experts > 1024 || c->n_groups > 32) return MOE_ERR_UNSUPPORTED;
  if (c->act_dtype == MOE_F32 && c->router_dtype == MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (c->n_shared > 0 && (c->n_heads != 1 || c->latent_proj)) return MOE_ERR_UNSUPPORTED;
  if (ec && (c->n_heads != 1 || c->n_groups || c->latent_proj)) return MOE_ERR_UNSUPPORTED;
  if (c->seq_len > 0 && c->n_heads != 1) return MOE_ERR_UNSUPPORTED;
  const long kslots = ec ? c->n_experts : (long)c->n_heads * c->top_k;
  if ((long)c->T * kslots > 0x7FFFFFFFL) return MOE_ERR_UNSUPPORTED;
  {
    // the GEMM addresses one group's operands with 32-bit element offsets
    const long lim = 1L << 31, T = c->T, D = (long)c->n_heads * c->d_head, fs = (long)c->n_shared * c->d_ff;
    const long m = c->act == MOE_ACT_SWIGLU ? 2 : 1;
    if (T * std::max<long>({(long)c->d_model, D, m * c->d_ff, m * fs}) >= lim) return MOE_ERR_UNSUPPORTED;
    if ((long)c->d_ff * c->d_head >= lim || fs * c->d_model >= lim || D * c->d_model >= lim)
      return MOE_ERR_UNSUPPORTED;
  }
  s->T = c->T; s->d = c->d_model; s->H = c->n_heads; s->dh = c->d_head; s->E = c->n_experts; s->Eh = Eh;
  s->k = ec ? Eh : c->top_k; s->K = (int)kslots;
  s->n_groups = c->n_groups; s->topk_groups = c->topk_groups; s->renorm = c->renorm;
  s->drop = ec ? moe::DROP_TOPC : c->drop; s->C = c->capacity; s->keep_num = c->keep_num;
  s->keep_den = c->keep_den;
  s->expert_choice = ec; s->sel_gate = c->sel_bias_gate; s->seq_len = c->seq_len;
  s->dff = c->d_ff; s->act = c->act; s->n_shared = c->n_shared; s->latent = c->latent_proj;
  s->residual = c->residual;
  s->act_f32 = c->act_dtype == MOE_F32;
  s->router_f32 = c->router_dtype == MOE_F32;
  long tk = (long)s->T * s->K;
  if (ec) s->R_max = (long)s->E * std::min<long>(s->C, s->T);
  else s->R_max = (s->drop == MOE_DROP_CAPACITY) ? std::min<long>(tk, (long)s->E * s->C) : tk;
  if (!moe::route_supported(*s)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t scratch_bytes(const Shape &s) {
  size_t m = moe::route_ws_bytes(s);
  size_t v = moe::dispatch_ws_bytes(s);
  if (v > m) m = v;
  v = moe::dispatch_after_route_ws_bytes(s);  // the layer's dispatch keeps the router's counts
  if (v > m) m = v;
  v = moe::ffn_ws_bytes(s);
  if (v > m) m = v;
  v = moe::dense_ws_bytes();
  if (v > m) m = v;
  return m;
}

// intermediates of moe_layer_fwd, in workspace order
struct LayerBufs {
  size_t topk_idx, topk_w, demand, counts, offsets, row_of, src_of, aux, z, y_perm, shared, o, scratch, total;
};

LayerBufs layer_layout(const Shape &s) {
  const size_t esz = s.act_f32 ? 4 : 2;
  const size_t tk = (size_t)s.T * s.K;
  LayerBufs b{};
  size_t o = 0;
  b.topk_idx = o; o += al(tk * 4);
  b.topk_w = o; o += al(tk * 4);
  b.demand = o; o += al((size_t)s.E * 4);
  b.counts = o; o += al((size_t)s.E * 4);
  b.offsets = o; o += al((size_t)(s.E + 1) * 4);
  b.row_of = o; o += al(tk * 4);
  b.src_of = o; o += al((size_t)s.R_max * 4);
  b.aux = o; o += al(4);
  b.z = o; o += s.latent ? al((size_t)s.T * s.H * s.dh * esz) : 0;
  b.y_perm = o; o += al((size_t)s.R_max * s.dh * esz);
  b.shared = o; o += s.n_shared ? al((size_t)s.T * s.d * esz) : 0;
  b.o = o; o += s.latent ? al((size_t)s.T * s.H * s.dh * esz) : 0;
  b.scratch = o; o += scratch_bytes(s);
  b.total = o;
  return b;
}

int check_ws(const Shape &s, const void *ws, size_t ws_bytes) {
  if (!ws || ((uintptr_t)ws & 255)) return MOE_ERR_WORKSPACE;
  if (ws_bytes < layer_layout(s).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// HIP's last-error state also holds errors of earlier, unrelated runtime
// calls of the caller; clear it before our first launch so that the checks
// after each launch see only our own launches
void clear_stale_error() { (void)hipGetLastError(); }

// the gathered operand rows are addressed with 32-bit element offsets into x
bool gather_supported(const Shape &s) { return (long)s.T * s.H * s.dh < (1L << 31); }

int rc_of(int launcher_rc) {
  if (launcher_rc == -2) return MOE_ERR_UNSUPPORTED;
  if (launcher_rc != 0) return MOE_ERR_HIP;
  return MOE_OK;
}

// ---------------------------------------------------------------- backward
// columns of the per-expert padded, transposed activations: every expert's
// rows rounded up to 64 (the GEMM k-chunk), and a multiple of 64 overall so
// rows of the transposed buffers stay 16-byte aligned
long rpad_bound(const Shape &s) { return (s.R_max + 63) / 64 * 64 + 64L * s.E; }
long tpad(const Shape &s) { return (s.T + 63) / 64 * 64; }

// The weight-gradient products address their transposed operands with 32-bit
// element offsets: every transposed buffer must stay below 2^31 elements.
bool bwd_supported(const Shape &s) {
  const long m = s.act == MOE_ACT_SWIGLU ? 2 : 1, lim = 1L << 31;
  const long rows = std::max<long>(s.dh, m * s.dff);
  if (!gather_supported(s) || rows * rpad_bound(s) >= lim) return false;
  const long wide = std::max<long>({(long)s.d, (long)s.H * s.dh, m * s.n_shared * (long)s.dff});
  return wide * tpad(s) < lim;
}

struct BwdBufs {
  size_t dg, dl, rpart, rplanes, seqcnt, dY, dH, dAB, Hr, dXr, poff, pmap_r, pmap_x, Xt, dYt, dABt, Ht, prefix, kwin;
  size_t dHs, dABs, Hs, dxs, dyt, xt, dABst, Hst, dout, du, ot, dut, spart, epart, kwsplit, total;
};

BwdBufs bwd_layout(const Shape &s) {
  const size_t esz = s.act_f32 ? 4 : 2, m = s.act == MOE_ACT_SWIGLU ? 2 : 1;
  const size_t R = s.R_max, Rp = rpad_bound(s), Tp = tpad(s), fs = (size_t)s.n_shared * s.dff;
  BwdBufs b{};
  size_t o = 0;
  b.dg = o; o += al((size_t)s.T * s.K * 4);
  b.dl = o; o += al((size_t)s.T * s.E * 4);
  b.rpart = o; o += al(moe::router_part_floats(s) * 4);
  b.rplanes = o; o += al(moe::router_planes_bytes(s));
  b.seqcnt = o; o += s.seq_len > 0 ? al((size_t)(s.T / s.seq_len) * s.E * 4) : 0;
  b.dY = o; o += al(R * s.dh * esz);
  b.dH = o; o += al(R * s.dff * esz);
  b.dAB = o; o += al(R * m * s.dff * esz);
  b.Hr = o; o += al(R * s.dff * esz);
  b.dXr = o; o += al(R * s.dh * esz);
  b.poff = o; o += al((size_t)(s.E + 1) * 4);
  b.pmap_r = o; o += al(Rp * 4);
  b.pmap_x = o; o += al(Rp * 4);
  b.Xt = o; o += al((size_t)s.dh * Rp * esz);
  b.dYt = o; o += al((size_t)s.dh * Rp * esz);
  b.dABt = o; o += al(m * s.dff * Rp * esz);
  b.Ht = o; o += al((size_t)s.dff * Rp * esz);
  b.prefix = o; o += al((size_t)2 * (s.E + 2) * 4);
  b.kwin = o; o += al(16 * 4);
  if (fs) {
    b.dHs = o; o += al((size_t)s.T * fs * esz);
    b.dABs = o; o += al((size_t)s.T * m * fs * esz);
    b.Hs = o; o += al((size_t)s.T * fs * esz);
    b.dxs = o; o += al((size_t)s.T * s.d * esz);
    b.dyt = o; o += al((size_t)s.d * Tp * esz);
    b.xt = o; o += al((size_t)s.d * Tp * esz);
    b.dABst = o; o += al(m * fs * Tp * esz);
    b.Hst = o; o += al(fs * Tp * esz);
  }
  // float32 partials of the split-K one-group products (shared experts, projections)
  {
    size_t mx = 0;
    auto need = [&](long M, long N) {
      mx = std::max(mx, (size_t)moe::splitk_count(s.act_f32, (int)M, (int)N, Tp) * M * N * 4);
    };
    if (fs) {
      need(s.d, fs);
      need(fs, s.d);
    }
    if (s.latent) {
      need(s.d, (long)s.H * s.dh);
      need((long)s.H * s.dh, s.d);
    }
    b.spart = o; o += al(mx);
    // the per-expert weight gradients: windows cut in pieces of bounded depth,
    // float32 partials for the pieces of cut windows
    const int d2 = moe::kgroup_piece_depth(s.act_f32, s.E, s.dh, s.dff, Rp);
    const int d1 = moe::kgroup_piece_depth(s.act_f32, s.E, s.dff, s.dh, Rp);
    const int dmin = std::min(d1, d2);
    b.epart = o; o += al((size_t)moe::kgroup_max_slots(Rp, dmin) * s.dh * s.dff * 4);
    b.kwsplit = o; o += al(((size_t)4 * moe::kgroup_max_pieces(s.E, Rp, dmin) + 1 + 2 * (size_t)s.E) * 4);
  }
  if (s.latent) {  // the projections: do, du and the transposes of dy, x, o, du
    const size_t D = (size_t)s.H * s.dh;
    b.dout = o; o += al((size_t)s.T * D * esz);
    b.du = o; o += al((size_t)s.T * D * esz);
    b.dyt = o; o += al((size_t)s.d * Tp * esz);
    b.xt = o; o += al((size_t)s.d * Tp * esz);
    b.ot = o; o += al(D * Tp * esz);
    b.dut = o; o += al(D * Tp * esz);
  }
  b.total = o;
  return b;
}

}  // namespace

// Every device pointer must be 16-byte aligned: the kernels move 16-byte
// vectors (direct global->LDS loads, row copies, combine).  NULL passes.
static bool misaligned(std::initializer_list<const void *> ps) {
  for (const void *p : ps)
    if ((uintptr_t)p & 15) return true;
  return false;
}
static bool misaligned_w(const moe_weights *w) {
  return misaligned({w->w_router, w->router_bias, w->w1, w->w3, w->w2, w->ws1, w->ws3, w->ws2, w->w_in, w->w_out,
                     w->sel_bias});
}
static bool misaligned_wt(const moe_weights_t *t) {
  return misaligned({t->w13t, t->w2t, t->ws13t, t->ws2t, t->w_in_t, t->w_out_t});
}
static bool misaligned_io(const moe_layer_io *io) {
  return misaligned({io->logits, io->topk_idx, io->topk_w, io->demand, io->counts, io->offsets, io->row_of,
                     io->src_of, io->aux_loss, io->seq_loss, io->z, io->x_perm, io->y_perm, io->shared_out, io->o,
                     io->gu});
}
static bool misaligned_g(const moe_grads *g) {
  return misaligned({g->dx, g->dw_router, g->dbias, g->dw1, g->dw3, g->dw2, g->dws1, g->dws3, g->dws2, g->dw_in,
                     g->dw_out});
}

extern "C" {

size_t moe_workspace_bytes(const moe_config *cfg) {
  Shape s;
  if (make_shape(cfg, &s) != MOE_OK) return 0;
  return layer_layout(s).total;
}

int64_t moe_rows_upper_bound(const moe_config *cfg) {
  Shape s;
  if (make_shape(cfg, &s) != MOE_OK) return -1;
  return s.R_max;
}

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_ARG: return "MOE_ERR_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: valid request outside the supported shapes";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small or not 256-byte aligned";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    default: return "unknown moe_status";
  }
}

int moe_check_config(const moe_config *cfg) {
  Shape s;
  return make_shape(cfg, &s);
}

int moe_route(const moe_config *cfg, const void *x, const void *w_router, const float *bias, float *logits, int mode,
              int32_t *topk_idx, float *topk_w, float *aux_loss, void *ws, size_t ws_bytes, hipStream_t stream) {
  return moe_route_ex(cfg, x, w_router, bias, nullptr, logits, mode, topk_idx, topk_w, aux_loss, nullptr, ws,
                      ws_bytes, stream);
}

int moe_route_ex(const moe_config *cfg, const void *x, const void *w_router, const float *bias,
                 const float *sel_bias, float *logits, int mode, int32_t *topk_idx, float *topk_w,
                 float *aux_loss, float *seq_loss, void *ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (mode < MOE_LOGITS_COMPUTE || mode > MOE_LOGITS_LOAD) return MOE_ERR_ARG;
  if (!topk_idx || !topk_w) return MOE_ERR_ARG;
  if (mode != MOE_LOGITS_LOAD && (!x || !w_router)) return MOE_ERR_ARG;
  if (mode != MOE_LOGITS_COMPUTE && !logits) return MOE_ERR_ARG;
  if (misaligned({x, w_router, bias, sel_bias, logits, topk_idx, topk_w, aux_loss, seq_loss})) return MOE_ERR_ARG;
  if (aux_loss && s.H != 1) return MOE_ERR_UNSUPPORTED;
  if (seq_loss && s.seq_len == 0) return MOE_ERR_ARG;
  if (sel_bias && s.expert_choice) return MOE_ERR_UNSUPPORTED;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  if (s.T == 0) return MOE_OK;
  clear_stale_error();
  return rc_of(moe::launch_route(s, x, w_router, bias, sel_bias, logits, mode, topk_idx, topk_w, aux_loss,
                                 seq_loss, ws, stream));
}

int moe_sel_bias_update(const moe_config *cfg, const int32_t *load, float *sel_bias, float gamma,
                        hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (!load || !sel_bias) return MOE_ERR_ARG;
  if (misaligned({load, sel_bias})) return MOE_ERR_ARG;
  clear_stale_error();
  return rc_of(moe::launch_sel_bias_update(s, load, sel_bias, gamma, stream));
}

int moe_dispatch(const moe_config *cfg, const int32_t *topk_idx, const float *topk_w, const void *x,
                 int32_t *demand, int32_t *counts, int32_t *offsets, int32_t *row_of, int32_t *src_of, void *x_perm,
                 void *ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (!topk_idx || !demand || !counts || !offsets || !row_of || (!src_of && s.R_max) || (x_perm && !x))
    return MOE_ERR_ARG;
  if (s.drop >= moe::DROP_AFFINITY && !topk_w) return MOE_ERR_ARG;  // affinity keep and expert choice read gates
  if (misaligned({topk_idx, topk_w, x, demand, counts, offsets, row_of, src_of, x_perm})) return MOE_ERR_ARG;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  if (s.T == 0) return MOE_OK;
  clear_stale_error();
  return rc_of(moe::launch_dispatch(s, topk_idx, topk_w, x, demand, counts, offsets, row_of, src_of, x_perm, ws,
                                    stream));
}

int moe_dispatch_noalloc(const moe_config *cfg, const int32_t *topk_idx, const float *topk_w, const void *x,
                         int32_t *demand, int32_t *counts, int32_t *offsets, int32_t *row_of, int32_t *src_of,
                         void *x_perm, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (!topk_idx || !demand || !counts || !offsets || !row_of || (!src_of && s.R_max) || (x_perm && !x))
    return MOE_ERR_ARG;
  if (s.drop >= moe::DROP_AFFINITY && !topk_w) return MOE_ERR_ARG;
  if (misaligned({topk_idx, topk_w, x, demand, counts, offsets, row_of, src_of, x_perm})) return MOE_ERR_ARG;
  if (moe::dispatch_ws_bytes(s) > moe::DISPATCH_SCRATCH_MAX) {
    if (getenv("MOE_DEBUG"))
      fprintf(stderr, "moe: moe_dispatch_noalloc needs %zu bytes of scratch, the library holds %zu\n",
              moe::dispatch_ws_bytes(s), moe::DISPATCH_SCRATCH_MAX);
    return MOE_ERR_WORKSPACE;
  }
  if (s.T == 0) return MOE_OK;
  void *scr = nullptr;
  if (moe::dispatch_scratch(&scr)) return MOE_ERR_HIP;
  clear_stale_error();
  return rc_of(moe::launch_dispatch(s, topk_idx, topk_w, x, demand, counts, offsets, row_of, src_of, x_perm, scr,
                                    stream));
}

int moe_check_topk(const moe_config *cfg, const int32_t *topk_idx, int32_t *status, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (!status || (!topk_idx && s.T)) return MOE_ERR_ARG;
  if (misaligned({topk_idx, status})) return MOE_ERR_ARG;
  clear_stale_error();
  return rc_of(moe::launch_topk_check(s, topk_idx, status, stream));
}

int moe_expert_ffn(const moe_config *cfg, const void *x_perm, const int32_t *offsets, const void *w1, const void *w3,
                   const void *w2, void *y_perm, const void *x_shared, const void *ws1, const void *ws3,
                   const void *ws2, void *shared_out, void *ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (((!x_perm || !y_perm) && s.R_max) || !offsets || !w1 || !w2) return MOE_ERR_ARG;
  if (misaligned({x_perm, offsets, w1, w3, w2, y_perm, x_shared, ws1, ws3, ws2, shared_out})) return MOE_ERR_ARG;
  if ((s.act == MOE_ACT_SWIGLU) != (w3 != nullptr)) return MOE_ERR_ARG;
  if (s.n_shared) {
    if (!x_shared || !ws1 || !ws2 || !shared_out) return MOE_ERR_ARG;
    if ((s.act == MOE_ACT_SWIGLU) != (ws3 != nullptr)) return MOE_ERR_ARG;
  }
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  if (s.T == 0) return MOE_OK;
  clear_stale_error();
  return rc_of(moe::launch_expert_ffn(s, x_perm, nullptr, offsets, w1, w3, w2, y_perm, x_shared, ws1, ws3, ws2,
                                      shared_out, ws, stream));
}

int moe_expert_ffn_gather(const moe_config *cfg, const void *x, const int32_t *src_of, const int32_t *offsets,
                          const void *w1, const void *w3, const void *w2, void *y_perm, const void *x_shared,
                          const void *ws1, const void *ws3, const void *ws2, void *shared_out, void *ws,
                          size_t ws_bytes, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (((!x || !src_of || !y_perm) && s.R_max) || !offsets || !w1 || !w2) return MOE_ERR_ARG;
  if (misaligned({x, src_of, offsets, w1, w3, w2, y_perm, x_shared, ws1, ws3, ws2, shared_out})) return MOE_ERR_ARG;
  if ((s.act == MOE_ACT_SWIGLU) != (w3 != nullptr)) return MOE_ERR_ARG;
  if (s.n_shared) {
    if (!x_shared || !ws1 || !ws2 || !shared_out) return MOE_ERR_ARG;
    if ((s.act == MOE_ACT_SWIGLU) != (ws3 != nullptr)) return MOE_ERR_ARG;
  }
  if (!gather_supported(s)) return MOE_ERR_UNSUPPORTED;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  if (s.T == 0) return MOE_OK;
  clear_stale_error();
  return rc_of(moe::launch_expert_ffn(s, x, src_of, offsets, w1, w3, w2, y_perm, x_shared, ws1, ws3, ws2,
                                      shared_out, ws, stream));
}

int moe_combine(const moe_config *cfg, const void *y_perm, const int32_t *row_of, const float *topk_w,
                const void *residual, const void *shared_out, void *y, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if ((!y_perm && s.R_max) || !row_of || !topk_w || !y) return MOE_ERR_ARG;
  if (misaligned({y_perm, row_of, topk_w, residual, shared_out, y})) return MOE_ERR_ARG;
  if (s.T == 0) return MOE_OK;
  clear_stale_error();
  return rc_of(moe::launch_combine(s, y_perm, row_of, topk_w, residual, shared_out, y, stream));
}

int moe_layer_fwd(const moe_config *cfg, const moe_weights *w, const void *x, void *y, moe_layer_io *io, void *ws,
                  size_t ws_bytes, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  moe_layer_io none;
  memset(&none, 0, sizeof(none));
  if (!io) io = &none;
  const int mode = io->logits_mode;
  if (!w || !x || !y || x == y) return MOE_ERR_ARG;
  if (misaligned({x, y}) || misaligned_w(w) || misaligned_io(io)) return MOE_ERR_ARG;
  if (mode < MOE_LOGITS_COMPUTE || mode > MOE_LOGITS_LOAD) return MOE_ERR_ARG;
  if (mode != MOE_LOGITS_COMPUTE && !io->logits) return MOE_ERR_ARG;
  if (mode != MOE_LOGITS_LOAD && !w->w_router) return MOE_ERR_ARG;
  if (!w->w1 || !w->w2 || ((s.act == MOE_ACT_SWIGLU) != (w->w3 != nullptr))) return MOE_ERR_ARG;
  if (s.n_shared && (!w->ws1 || !w->ws2 || ((s.act == MOE_ACT_SWIGLU) != (w->ws3 != nullptr)))) return MOE_ERR_ARG;
  if (s.latent && (!w->w_in || !w->w_out)) return MOE_ERR_ARG;
  if (io->aux_loss && s.H != 1) return MOE_ERR_UNSUPPORTED;
  if (io->seq_loss && s.seq_len == 0) return MOE_ERR_ARG;
  if (w->sel_bias && s.expert_choice) return MOE_ERR_UNSUPPORTED;
  if (!io->x_perm && !gather_supported(s)) return MOE_ERR_UNSUPPORTED;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  if (s.T == 0) return MOE_OK;

  const LayerBufs L = layer_layout(s);
  char *base = (char *)ws;
  auto pick = [&](void *user, size_t off) -> void * { return user ? user : (void *)(base + off); };
  int32_t *topk_idx = (int32_t *)pick(io->topk_idx, L.topk_idx);
  float *topk_w = (float *)pick(io->topk_w, L.topk_w);
  int32_t *demand = (int32_t *)pick(io->demand, L.demand);
  int32_t *counts = (int32_t *)pick(io->counts, L.counts);
  int32_t *offsets = (int32_t *)pick(io->offsets, L.offsets);
  int32_t *row_of = (int32_t *)pick(io->row_of, L.row_of);
  int32_t *src_of = (int32_t *)pick(io->src_of, L.src_of);
  void *x_perm = io->x_perm;  // NULL: the expert FFN gathers rows from xin
  void *y_perm = pick(io->y_perm, L.y_perm);
  void *shared = s.n_shared ? pick(io->shared_out, L.shared) : nullptr;
  void *z = s.latent ? pick(io->z, L.z) : nullptr;
  void *o = s.latent ? pick(io->o, L.o) : nullptr;
  void *scratch = base + L.scratch;

  clear_stale_error();
  const void *xin = x;  // router and expert input
  if (s.latent) {
    if ((rc = rc_of(moe::launch_dense(s.act_f32, x, w->w_in, z, nullptr, s.T, s.H * s.dh, s.d, scratch, stream))))
      return rc;
    xin = z;
  }
  // the router's per-block choice counts are the histogram dispatch needs: no histogram launch
  int32_t *route_hist = (int32_t *)((char *)scratch + moe::route_hist_offset(s));
  if ((rc = rc_of(moe::launch_route(s, xin, w->w_router, w->router_bias, w->sel_bias, io->logits, mode, topk_idx,
                                    topk_w, io->aux_loss, io->seq_loss, scratch, stream, route_hist))))
    return rc;
  if ((rc = rc_of(moe::launch_dispatch(s, topk_idx, topk_w, xin, demand, counts, offsets, row_of, src_of, x_perm,
                                       scratch, stream, s.expert_choice ? nullptr : route_hist))))
    return rc;
  // Where every (token, head) keeps its one choice (multi-head latent, top-1
  // per head, nothing dropped), the expert FFN's epilogue writes each row,
  // gated, straight into its slice of o: the combine pass (a read of y_perm
  // and a write of o) is not run, and y_perm is written only when the caller
  // asks for it.  o is bitwise what the combine would write.
  const bool fold = moe::fold_supported(s);
  moe::FoldOut fo{};
  if (fold) fo = moe::FoldOut{o, topk_w, src_of};
  // the routed pre-activations, kept for the backward when the caller gives a buffer
  void *gsave = (io && io->gu && moe::ffn_grouped(s)) ? io->gu : nullptr;
  if ((rc = rc_of(moe::launch_expert_ffn(s, x_perm ? x_perm : xin, x_perm ? nullptr : src_of, offsets, w->w1,
                                         w->w3, w->w2, (fold && !io->y_perm) ? nullptr : y_perm, x, w->ws1, w->ws3,
                                         w->ws2, shared, scratch, stream, fo, gsave))))
    return rc;
  const void *res = (!s.latent && s.residual) ? x : nullptr;
  if (!fold && (rc = rc_of(moe::launch_combine(s, y_perm, row_of, topk_w, res, shared, s.latent ? o : y, stream))))
    return rc;
  if (s.latent) {
    if ((rc = rc_of(moe::launch_dense(s.act_f32, o, w->w_out, y, x, s.T, s.d, s.H * s.dh, scratch, stream))))
      return rc;
  }
  return MOE_OK;
}

size_t moe_backward_workspace_bytes(const moe_config *cfg) {
  Shape s;
  if (make_shape(cfg, &s) != MOE_OK || !bwd_supported(s)) return 0;
  return bwd_layout(s).total;
}

int moe_transpose_weights(const moe_config *cfg, const moe_weights *w, const moe_weights_t *wt, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (!w || !wt || !w->w1 || !w->w2 || !wt->w13t || !wt->w2t) return MOE_ERR_ARG;
  if (misaligned_w(w) || misaligned_wt(wt)) return MOE_ERR_ARG;
  const bool glu = s.act == MOE_ACT_SWIGLU;
  if (glu && !w->w3) return MOE_ERR_ARG;
  if (s.n_shared && (!w->ws1 || !w->ws2 || (glu && !w->ws3) || !wt->ws13t || !wt->ws2t)) return MOE_ERR_ARG;
  if (s.latent && (!w->w_in || !w->w_out || !wt->w_in_t || !wt->w_out_t)) return MOE_ERR_ARG;
  const long m = glu ? 2 : 1, esz = s.act_f32 ? 4 : 2, dff = s.dff, dh = s.dh;
  clear_stale_error();
  if (s.latent) {
    const long D = (long)s.H * dh, d = s.d;
    // w_in_t [d][D] = W_in^T, w_out_t [D][d] = W_out^T
    if ((rc = rc_of(moe::launch_transpose(s.act_f32, w->w_in, d, 0, nullptr, D, D, (int)d, 0, wt->w_in_t, D, 0, 1,
                                          stream))))
      return rc;
    if ((rc = rc_of(moe::launch_transpose(s.act_f32, w->w_out, D, 0, nullptr, d, d, (int)D, 0, wt->w_out_t, d, 0, 1,
                                          stream))))
      return rc;
  }
  // w13t[e][c][0..dff) = W1[e][..][c], [dff..2dff) = W3[e][..][c]
  if ((rc = rc_of(moe::launch_transpose(s.act_f32, w->w1, dh, dff * dh, nullptr, dff, dff, (int)dh, 0, wt->w13t,
                                        m * dff, dh * m * dff, s.E, stream))))
    return rc;
  if (glu && (rc = rc_of(moe::launch_transpose(s.act_f32, w->w3, dh, dff * dh, nullptr, dff, dff, (int)dh, 0,
                                               (char *)wt->w13t + dff * esz, m * dff, dh * m * dff, s.E, stream))))
    return rc;
  if ((rc = rc_of(moe::launch_transpose(s.act_f32, w->w2, dff, dh * dff, nullptr, dh, dh, (int)dff, 0, wt->w2t, dh,
                                        dff * dh, s.E, stream))))
    return rc;
  if (s.n_shared) {
    const long fs = (long)s.n_shared * dff, d = s.d;
    if ((rc = rc_of(moe::launch_transpose(s.act_f32, w->ws1, d, 0, nullptr, fs, fs, (int)d, 0, wt->ws13t, m * fs,
                                          0, 1, stream))))
      return rc;
    if (glu && (rc = rc_of(moe::launch_transpose(s.act_f32, w->ws3, d, 0, nullptr, fs, fs, (int)d, 0,
                                                 (char *)wt->ws13t + fs * esz, m * fs, 0, 1, stream))))
      return rc;
    if ((rc = rc_of(moe::launch_transpose(s.act_f32, w->ws2, fs, 0, nullptr, d, d, (int)fs, 0, wt->ws2t, d, 0, 1,
                                          stream))))
      return rc;
  }
  return MOE_OK;
}

int moe_layer_bwd(const moe_config *cfg, const moe_weights *w, const moe_weights_t *wt, const void *x,
                  const void *dy, float aux_weight, float seq_weight, const moe_layer_io *io, moe_grads *g,
                  void *ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (!w || !wt || !x || !dy || !io || !g) return MOE_ERR_ARG;
  if (misaligned({x, dy}) || misaligned_w(w) || misaligned_wt(wt) || misaligned_io(io) || misaligned_g(g))
    return MOE_ERR_ARG;
  if (!bwd_supported(s)) return MOE_ERR_UNSUPPORTED;
  // a bias inside renormalised gates changes the renormalisation's derivative
  if (w->sel_bias && s.sel_gate && s.renorm) return MOE_ERR_UNSUPPORTED;
  const bool glu = s.act == MOE_ACT_SWIGLU;
  if (!w->w_router || !w->w1 || !w->w2 || (glu && !w->w3) || !wt->w13t || !wt->w2t) return MOE_ERR_ARG;
  if (!io->logits || !io->topk_idx || !io->topk_w || !io->demand || !io->offsets || !io->row_of ||
      ((!io->src_of || !io->y_perm) && s.R_max))
    return MOE_ERR_ARG;
  if (!g->dx || !g->dw_router || !g->dw1 || !g->dw2 || (glu && !g->dw3)) return MOE_ERR_ARG;
  if (s.n_shared && (!w->ws1 || !w->ws2 || (glu && !w->ws3) || !wt->ws13t || !wt->ws2t || !g->dws1 || !g->dws2 ||
                     (glu && !g->dws3)))
    return MOE_ERR_ARG;
  if (s.latent && (!w->w_in || !w->w_out || !wt->w_in_t || !wt->w_out_t || !io->z || !io->o || !g->dw_in ||
                   !g->dw_out))
    return MOE_ERR_ARG;
  // the aux loss is defined for one routing head
  if (s.H > 1 && aux_weight != 0.0f) return MOE_ERR_UNSUPPORTED;
  if (seq_weight != 0.0f && s.seq_len == 0) return MOE_ERR_ARG;
  const BwdBufs L = bwd_layout(s);
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (s.T == 0) return MOE_OK;

  char *base = (char *)ws;
  auto at = [&](size_t off) { return (void *)(base + off); };
  float *dg = (float *)at(L.dg), *dl = (float *)at(L.dl);
  void *dY = at(L.dY), *dH = at(L.dH), *dAB = at(L.dAB), *Hr = at(L.Hr), *dXr = at(L.dXr);
  int32_t *poff = (int32_t *)at(L.poff), *pmap_r = (int32_t *)at(L.pmap_r), *pmap_x = (int32_t *)at(L.pmap_x);
  void *Xt = at(L.Xt), *dYt = at(L.dYt), *dABt = at(L.dABt), *Ht = at(L.Ht);
  int32_t *prefix = (int32_t *)at(L.prefix), *kwin = (int32_t *)at(L.kwin);
  const bool f32 = s.act_f32;
  const long m = glu ? 2 : 1, esz = f32 ? 4 : 2, dh = s.dh, dff = s.dff, d = s.d, Rp = rpad_bound(s), Tp = tpad(s);
  const long D = (long)s.H * dh;                 // width of the expert input u (x, or the latent z)
  const void *u = s.latent ? io->z : x;
  const int epi_bwd = glu ? moe::GEMM_EPI_SWIGLU_BWD : moe::GEMM_EPI_RELU_BWD;
  const int32_t *offsets = io->offsets, *src_of = io->src_of;
  // one group's C[M, N] = A B^T over the T (padded) tokens: A [M][Tp], B [N][Tp],
  // k-chunked with arows and brows rows
  auto tokens_product = [&](const void *A, long arows, const void *B, long brows, void *C, int M, int N) -> int {
    const int S = moe::splitk_count(f32, M, N, Tp);
    if (int r = rc_of(moe::launch_set_kwin(kwin, (int)Tp, S, stream))) return r;
    return rc_of(moe::gemm_splitk(f32, A, arows, B, brows, C, M, N, S, kwin, (float *)at(L.spart), stream));
  };
  const long KC = 128 / esz;  // elements per k-chunk of the transposed buffers

  clear_stale_error();
  // latent layer: the gradient of o is do = dy W_out
  const void *dyo = dy;
  if (s.latent) {
    dyo = at(L.dout);
    if ((rc = rc_of(moe::launch_dense(f32, dy, wt->w_out_t, at(L.dout), nullptr, s.T, (int)D, (int)d, nullptr,
                                      stream))))
      return rc;
  }
  // gate gradients dg = <do_h, y_perm>, scaled row gradients dY = g * do_h
  if ((rc = rc_of(moe::launch_bwd_rows(s, dyo, D, io->y_perm, io->topk_w, src_of, io->topk_idx, offsets, dY, dg,
                                       stream))))
    return rc;
  if ((rc = rc_of(moe::launch_bwd_pad(s, offsets, src_of, poff, pmap_r, pmap_x, Rp, stream)))) return rc;
  // dH = dY W2  (B = W2^T rows)
  if ((rc = rc_of(moe::gemm_routed(s, moe::GEMM_EPI_PLAIN, dY, dh, nullptr, wt->w2t, nullptr, dh, dff * dh, dH, dff,
                                   (int)dff, (int)dh, offsets, nullptr, 0, nullptr, 0, prefix, stream))))
    return rc;
  if (io->gu && moe::ffn_grouped(s)) {
    // dA|dB and H from the pre-activations the forward kept
    if ((rc = rc_of(moe::launch_bwd_saved_act(s, io->gu, dH, dAB, Hr, offsets, stream)))) return rc;
  } else {
    // recompute the gate/up products from u, with the backward epilogue: dA|dB, H
    if ((rc = rc_of(moe::gemm_routed(s, epi_bwd, u, D, src_of, w->w1, glu ? w->w3 : nullptr, dh, dff * dh, dAB,
                                     m * dff, (int)dff, (int)dh, offsets, dH, dff, Hr, dff, prefix, stream))))
      return rc;
  }
  // dX rows = [dA dB] [W1; W3]
  if ((rc = rc_of(moe::gemm_routed(s, moe::GEMM_EPI_PLAIN, dAB, m * dff, nullptr, wt->w13t, nullptr, m * dff,
                                   dh * m * dff, dXr, dh, (int)dh, (int)(m * dff), offsets, nullptr, 0, nullptr, 0,
                                   prefix, stream))))
    return rc;
  // transposed, per-expert padded activations for the weight gradients
  // (u viewed as [T*H, dh]: pmap_x holds t*H + h)
  if ((rc = rc_of(moe::launch_transpose(f32, u, dh, 0, pmap_x, 0, Rp, (int)dh, 0, Xt, dh, 0, 1, stream, 1))))
    return rc;
  if ((rc = rc_of(moe::launch_transpose(f32, dY, dh, 0, pmap_r, 0, Rp, (int)dh, 0, dYt, dh, 0, 1, stream, 1))))
    return rc;
  if ((rc = rc_of(moe::launch_transpose(f32, dAB, m * dff, 0, pmap_r, 0, Rp, (int)(m * dff), 0, dABt, m * dff, 0, 1,
                                        stream, 1))))
    return rc;
  if ((rc = rc_of(moe::launch_transpose(f32, Hr, dff, 0, pmap_r, 0, Rp, (int)dff, 0, Ht, dff, 0, 1, stream, 1))))
    return rc;
  // dW2_e = dY_e^T H_e, dW1_e = dA_e^T X_e, dW3_e = dB_e^T X_e (windows split when
  // the experts' output tiles alone would not fill the chip)
  // (each expert's window cut in pieces of bounded depth, so one hot expert
  // does not leave the chip idle while its tiles contract every row)
  auto expert_wgrad = [&](const void *A, long arows, const void *B, long brows, void *C, long ldc, int M,
                          int N) -> int {
    const int depth = moe::kgroup_piece_depth(f32, s.E, M, N, Rp);
    const long maxp = moe::kgroup_max_pieces(s.E, Rp, depth);
    int32_t *tab = (int32_t *)at(L.kwsplit);
    return rc_of(moe::gemm_kgrouped_pieces(f32, A, arows, B, brows, C, ldc, (long)M * N, s.E, M, N, poff, depth,
                                           maxp, tab, tab + 4 * maxp + 1, (float *)at(L.epart), stream));
  };
  if ((rc = expert_wgrad(dYt, dh, Ht, dff, g->dw2, dff, (int)dh, (int)dff))) return rc;
  if ((rc = expert_wgrad(dABt, m * dff, Xt, dh, g->dw1, dh, (int)dff, (int)dh))) return rc;
  if (glu && (rc = expert_wgrad((char *)dABt + dff * KC * esz, m * dff, Xt, dh, g->dw3, dh, (int)dff, (int)dh)))
    return rc;
  // router: dl, dW_r, dbias
  int32_t *seqcnt = seq_weight != 0.0f ? (int32_t *)at(L.seqcnt) : nullptr;
  if (seqcnt && (rc = rc_of(moe::launch_seq_counts(s, io->topk_idx, seqcnt, stream)))) return rc;
  if ((rc = rc_of(moe::launch_router_bwd(s, io->logits, io->topk_idx, io->topk_w, dg, io->demand, aux_weight,
                                         seqcnt, seq_weight, u, dl, (uint16_t *)at(L.rplanes),
                                         (float *)at(L.rpart), g->dw_router, g->dbias, stream))))
    return rc;
  // shared experts: the same MLP backward over all T tokens with gate 1
  void *dxs = nullptr;
  if (s.n_shared) {
    const long fs = (long)s.n_shared * dff;
    void *dHs = at(L.dHs), *dABs = at(L.dABs), *Hs = at(L.Hs), *dyt = at(L.dyt), *xt = at(L.xt);
    void *dABst = at(L.dABst), *Hst = at(L.Hst);
    dxs = at(L.dxs);
    if ((rc = rc_of(moe::gemm_plain(f32, moe::GEMM_EPI_PLAIN, dy, d, wt->ws2t, nullptr, d, dHs, fs, s.T, (int)fs,
                                    (int)d, nullptr, 0, nullptr, 0, stream))))
      return rc;
    if ((rc = rc_of(moe::gemm_plain(f32, epi_bwd, x, d, w->ws1, glu ? w->ws3 : nullptr, d, dABs, m * fs, s.T,
                                    (int)fs, (int)d, dHs, fs, Hs, fs, stream))))
      return rc;
    if ((rc = rc_of(moe::gemm_plain(f32, moe::GEMM_EPI_PLAIN, dABs, m * fs, wt->ws13t, nullptr, m * fs, dxs, d, s.T,
                                    (int)d, (int)(m * fs), nullptr, 0, nullptr, 0, stream))))
      return rc;
    if ((rc = rc_of(moe::launch_transpose(f32, dy, d, 0, nullptr, s.T, Tp, (int)d, 0, dyt, d, 0, 1, stream, 1))))
      return rc;
    if ((rc = rc_of(moe::launch_transpose(f32, x, d, 0, nullptr, s.T, Tp, (int)d, 0, xt, d, 0, 1, stream, 1))))
      return rc;
    if ((rc = rc_of(moe::launch_transpose(f32, dABs, m * fs, 0, nullptr, s.T, Tp, (int)(m * fs), 0, dABst, m * fs, 0,
                                          1, stream, 1))))
      return rc;
    if ((rc = rc_of(moe::launch_transpose(f32, Hs, fs, 0, nullptr, s.T, Tp, (int)fs, 0, Hst, fs, 0, 1, stream, 1))))
      return rc;
    if ((rc = tokens_product(dyt, d, Hst, fs, g->dws2, (int)d, (int)fs))) return rc;
    if ((rc = tokens_product(dABst, m * fs, xt, d, g->dws1, (int)fs, (int)d))) return rc;
    if (glu && (rc = tokens_product((char *)dABst + fs * KC * esz, m * fs, xt, d, g->dws3, (int)fs, (int)d)))
      return rc;
  }
  if (!s.latent) {
    // dx = [dy] + [dxs] + sum_j dX rows + dl W_r (per head)
    return rc_of(moe::launch_bwd_dx(s, dy, dxs, dXr, io->row_of, dl, w->w_router, s.residual, g->dx, stream));
  }
  // latent layer: du as above, then dx = dy + du W_in, dW_in = du^T x, dW_out = dy^T o
  void *du = at(L.du), *dyt = at(L.dyt), *xt = at(L.xt), *ot = at(L.ot), *dut = at(L.dut);
  if ((rc = rc_of(moe::launch_bwd_dx(s, nullptr, nullptr, dXr, io->row_of, dl, w->w_router, 0, du, stream))))
    return rc;
  if ((rc = rc_of(moe::launch_dense(f32, du, wt->w_in_t, g->dx, dy, s.T, (int)d, (int)D, nullptr, stream))))
    return rc;
  if ((rc = rc_of(moe::launch_transpose(f32, dy, d, 0, nullptr, s.T, Tp, (int)d, 0, dyt, d, 0, 1, stream, 1))))
    return rc;
  if ((rc = rc_of(moe::launch_transpose(f32, x, d, 0, nullptr, s.T, Tp, (int)d, 0, xt, d, 0, 1, stream, 1))))
    return rc;
  if ((rc = rc_of(moe::launch_transpose(f32, io->o, D, 0, nullptr, s.T, Tp, (int)D, 0, ot, D, 0, 1, stream, 1))))
    return rc;
  if ((rc = rc_of(moe::launch_transpose(f32, du, D, 0, nullptr, s.T, Tp, (int)D, 0, dut, D, 0, 1, stream, 1))))
    return rc;
  if ((rc = tokens_product(dyt, d, ot, D, g->dw_out, (int)d, (int)D))) return rc;
  return tokens_product(dut, D, xt, d, g->dw_in, (int)D, (int)d);
}

}  // extern "C"

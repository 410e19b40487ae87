// Grouped GEMM for the expert FFN, on MFMA (bf16 in, float32 accumulate).
//
// Expert FFN: "MoE技术演进", "GShard" item 3 (W_o relu(W_i x), no biases) and
// "大语言模型并行策略（七）：专家并行", "MoE 模型的参数量分析" (SwiGLU experts: three
// d_model x d_moe matrices).  Shared experts are one more always-active group
// over all tokens: "MoE技术演进", "DeepSeekMoE" item 2.  The small batches per
// expert that the expert-parallelism page flags ("挑战三：计算不高效") are why all
// experts (and the shared group) run in ONE launch over a device-built tile
// list: a ragged expert with 11 rows costs one 128-row tile, not a launch.
//
// C[M_g, N] = A_g[M_g, K] * B_g[N, K]^T for groups g: routed expert e owns rows
// [offsets[e], offsets[e+1]) of A and C; an optional extra group (shared
// experts, or a plain dense product) has its own pointers and sizes.  Both
// operands are K-contiguous.  Tiles: 256 x 256 outputs with 8 waves (tall
// groups; a group's short tail goes to a second launch of 128 x 128 tiles, or
// 128 x 64 ones for narrow products) or
// 128 x 128 with 8 waves (SwiGLU: half the tile's B rows are gate rows, half
// up rows, so the output tile is BN/2 hidden columns wide); k-chunks of 128
// bytes per row in LDS rings with XOR-swizzled 16-byte slots, one barrier per
// k-chunk.  Waves whose rows lie past a group's end skip their MFMAs.
//
// What bounds it (measured on MI355X): with the global loads removed the MFMA
// + LDS-read loop runs at 75-85 % of the bf16 peak; the global -> LDS stream
// alone takes 70-90 % of the kernel's time.  Per 64-k chunk a 256 x 256 tile
// moves as many bytes through the LDS (fragment reads plus the direct-load
// writes) as its MFMAs take cycles at 128 bytes per clock, the rate the bank
// conflict counters point to; the 128 x 128 tiles move twice as many per
// MFMA and keep the MFMA pipes busy about half as often.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

// EPI_F32OUT: the plain product written in float32 (K-grouped mode only: the
// partial sums of a K-split product, added afterwards in a fixed order)
// EPI_PIECE: K-grouped pieces (pieces table): a whole window's product in the
// element type to its group's C block, a cut window's float32 partial to
// its slot of `part`
enum { EPI_PLAIN = 0, EPI_RELU = 1, EPI_SWIGLU = 2, EPI_RESID = 3, EPI_SWIGLU_BWD = 4, EPI_RELU_BWD = 5,
       EPI_F32OUT = 6, EPI_PIECE = 7 };
// epilogues whose B tile pairs gate rows with up rows (SwiGLU forward, and its backward)
static_assert(GEMM_EPI_PLAIN == EPI_PLAIN && GEMM_EPI_SWIGLU_BWD == EPI_SWIGLU_BWD &&
                  GEMM_EPI_RELU_BWD == EPI_RELU_BWD, "epilogue ids");
template <int EPI> constexpr bool kPair = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_BWD);

struct GemmArgs {
  const void *A; long lda;                    // routed: A rows indexed by offsets
  const int32_t *gather;                      // routed A row r = A[gather[r] / gK] + (e / gEh) * gdh, or NULL
  int gK, gEh, gdh;
  const void *B; const void *B2; long ldb; long bstride;
  void *C; long ldc;
  const int32_t *offsets;
  int E, N, K;
  const void *Ax; long ldax;                  // extra group
  const void *Bx; const void *Bx2; long ldbx;
  void *Cx; long ldcx;
  int Mx, Nx, Kx, has_x;
  long Mr_bound;                              // upper bound on the routed rows (sum over experts)
  const void *res; long ldres;                // EPI_RESID: added to the extra group's output
  const void *dh; long lddh;                  // *_BWD: upstream gradient of the hidden activation (rows as C)
  void *hout; long ldh;                       // *_BWD: the recomputed hidden activation (rows as C)
  const int32_t *kwin;                        // K-grouped mode: group g contracts columns [kwin[g], kwin[g+1])
  long cstride;                               //   of A and B; its C block at C + g * cstride.  A and B are
                                              //   k-chunked: element (row, k) at (k / KC) * ld * KC + row * KC
                                              //   + k % KC, KC = 128 bytes of elements, ld (lda, ldb) = the
                                              //   buffer's row count
  int Mk;                                     //   rows of A in that mode
  const int32_t *pieces;                      // K-grouped pieces: [npieces][4] = (group, k0, k1, slot or -1),
  const int32_t *npieces;                     //   the count on the device; slot >= 0: float32 partial at
  float *part;                                //   part + slot * M * N (row stride N), else C of the group
  const int32_t *prefix;                      // [G+1] tile prefix, or NULL: E == 0 and fixed_tiles tiles
  int fixed_tiles;
  int G;
  int split;  // 0: all rows of a group; 1: rows [0, cut); 2: rows [cut, M); 3, 4: see row_window
  void *gsave; long ldg;                      // EPI_SWIGLU / EPI_RELU, or NULL: the pre-activations (rows as
                                              //   C): SwiGLU gate g at [row][col], up u at [row][N + col]; ReLU a
};

// Rows of a group a launch covers.  With split launches, a group's rows are
// cut where its last 256-row tile would hold at most 128 rows: the head goes
// to 256-row tiles, the short tail to 128-row tiles in a second launch (a tail
// tile in the head launch would hold a CU for nearly as long as a full tile,
// since the tile's time goes to streaming its weight columns).
// A launch pair for groups of very unequal size (split 3 and 4): groups of
// at least SPLIT_HOT rows put their head in 256-row tiles (split 3), and the
// rest (their tails, and every row of the smaller groups) goes to 128-row
// tiles (split 4).
constexpr int SPLIT_BM = 256;
constexpr int SPLIT_HOT = 1024;
__host__ __device__ inline void row_window(int split, int M, int *beg, int *len) {
  const int rem = M % SPLIT_BM;
  const int cut = (rem == 0 || rem > SPLIT_BM / 2) ? M : M - rem;
  const bool hot = M >= SPLIT_HOT;
  if (split == 1) { *beg = 0; *len = cut; }
  else if (split == 2) { *beg = cut; *len = M - cut; }
  else if (split == 3) { *beg = 0; *len = hot ? cut : 0; }
  else if (split == 4) { *beg = hot ? cut : 0; *len = M - *beg; }
  else { *beg = 0; *len = M; }
}

template <int EPI, int BN_> __host__ __device__ inline int n_tiles(int N) {
  return kPair<EPI> ? (N + BN_ / 2 - 1) / (BN_ / 2) : (N + BN_ - 1) / BN_;
}

// Tile prefixes over groups for up to four launches at once (one block per
// launch): tiles_g = ceil(rows of g in the launch's window / bm) * nt_g.
struct PrepCfg {
  int bm, split, nt, ntx;  // row tile, row window, n-tiles of a routed / the extra group
};
struct PrepArgs {
  PrepCfg c[4];
  const int32_t *offsets;
  int E, has_x, Mx;
  int32_t *prefix;  // [launch][E + 2]
};

__global__ __launch_bounds__(1024) void gemm_prep_kernel(PrepArgs a) {
  __shared__ int s[1024];
  const PrepCfg c = a.c[blockIdx.x];
  int32_t *prefix = a.prefix + (size_t)blockIdx.x * (a.E + 2);
  const int E = a.E, G = E + a.has_x;
  const int tid = threadIdx.x;
  const int per = (G + 1023) / 1024;
  int loc[2] = {0, 0};
  int sum = 0;
  for (int i = 0; i < per && i < 2; ++i) {
    int g = tid * per + i;
    int v = 0;
    if (g < G) {
      int M = (g < E) ? a.offsets[g + 1] - a.offsets[g] : a.Mx;
      int beg;
      row_window(c.split, M, &beg, &M);
      v = (M + c.bm - 1) / c.bm * ((g < E) ? c.nt : c.ntx);
    }
    loc[i] = v;
    sum += v;
  }
  s[tid] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int u = (tid >= o) ? s[tid - o] : 0;
    __syncthreads();
    s[tid] += u;
    __syncthreads();
  }
  int run = s[tid] - sum;
  for (int i = 0; i < per && i < 2; ++i) {
    int g = tid * per + i;
    if (g < G) prefix[g] = run;
    run += loc[i];
  }
  if (tid == 1023) prefix[G] = s[1023];
}

// Tile BM x BN outputs (SwiGLU: BN/2 hidden columns, the B tile holding BN/2
// gate rows then BN/2 up rows); WGM x WGN waves, each (BM/WGM) x (BN/WGN);
// k-chunks of KS = 8 16-byte slots (128 B) per row.  The A and B chunks sit
// in rings of STA and STB LDS buffers, so the global loads of an operand run
// STA-1 (STB-1) chunks ahead of the MFMAs; the deeper ring goes to the
// operand whose loads miss L2 more.  Operands go global -> LDS with global_load_lds_dwordx4 (no VGPR
// staging): each wave instruction fills 64 consecutive 16-byte LDS slots, so
// every lane fetches the global chunk that belongs in its slot.  Slots are
// XOR-swizzled within a row so the 16 rows one ds_read_b128 touches fall in
// distinct banks.
// Four consecutive elements of a row as one access (the caller keeps them
// inside the row and 8-byte (bf16) / 16-byte (fp32) aligned).
template <typename TE> struct Quad;
template <> struct Quad<uint16_t> {
  using Raw = uint2;
  __device__ __forceinline__ static Raw raw(const uint16_t *p) { return *(const uint2 *)p; }
  __device__ __forceinline__ static void decode(const Raw u, float o[4]) {
    o[0] = bf16_to_f32((uint16_t)(u.x & 0xFFFFu)); o[1] = bf16_to_f32((uint16_t)(u.x >> 16));
    o[2] = bf16_to_f32((uint16_t)(u.y & 0xFFFFu)); o[3] = bf16_to_f32((uint16_t)(u.y >> 16));
  }
  __device__ __forceinline__ static void store(uint16_t *p, const float o[4]) {
    uint2 u;
    u.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
    u.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
    *(uint2 *)p = u;
  }
};
template <> struct Quad<float> {
  using Raw = float4;
  __device__ __forceinline__ static Raw raw(const float *p) { return *(const float4 *)p; }
  __device__ __forceinline__ static void decode(const Raw u, float o[4]) {
    o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w;
  }
  __device__ __forceinline__ static void store(float *p, const float o[4]) {
    *(float4 *)p = make_float4(o[0], o[1], o[2], o[3]);
  }
};

template <int KS>
__device__ __forceinline__ int swz(int row, int q) {
  static_assert(KS == 8, "128-byte k-chunks");
  return q ^ (row & 7);
}

template <typename TE, int EPI, int BM_, int BN_, int WGM, int WGN, int KS, int STA, int STB, bool SG>
__global__ __launch_bounds__(64 * WGM * WGN) void grouped_gemm_kernel(GemmArgs p) {
  constexpr int NT = 64 * WGM * WGN;    // threads
  constexpr int EPC = 16 / sizeof(TE);  // elements per 16-byte slot
  constexpr int BKE = KS * EPC;         // elements per k-chunk
  constexpr int WM = BM_ / WGM, WN = BN_ / WGN, MF = WM / 16, NF = WN / 16;
  constexpr int SA = BM_ * KS, SB = BN_ * KS;  // 16-byte slots per stage
  constexpr int LA = SA / NT, LB = SB / NT;    // slots per thread per stage
  constexpr int NKS = KS / 4;                  // MFMA k-steps per chunk
  static_assert(LA * NT == SA && LB * NT == SB, "tile / thread mismatch");
  static_assert(STA >= 2 && STB >= 2 && NKS == 2, "two k-steps per chunk, two or more stages");
  extern __shared__ u32x4 smem[];
  u32x4 *sA = smem;               // [STA][SA]
  u32x4 *sB = smem + STA * SA;    // [STB][SB]

  // tile count: the device-built prefix, or (no routed groups: a plain
  // product whose size the host knows) the fixed count
  const int tpg_k = p.kwin ? ((p.Mk + BM_ - 1) / BM_) * n_tiles<EPI, BN_>(p.N) : 0;
  const int total = p.prefix ? p.prefix[p.G] : (p.pieces ? *p.npieces * tpg_k : p.fixed_tiles);
  const int b = blockIdx.x;
  if (b >= total) return;
  // blocks go round-robin to the 8 XCDs; give each XCD a contiguous run of
  // tiles so tiles sharing operands share an L2
  // (K-grouped pieces: tiles of unequal depth, listed deepest first; they go
  // round-robin, so every XCD gets its share of each depth)
  const int q8 = total >> 3;
  const int lt = (b < 8 * q8 && !p.pieces) ? (b & 7) * q8 + (b >> 3) : b;
  int g = 0, local = lt;
  if (p.kwin) {
    // K-grouped: every group (or piece) has the same (Mk x N) tile grid
    g = lt / tpg_k;
    local = lt - g * tpg_k;
  } else if (p.prefix) {
    int lo = 0, hi = p.G - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (p.prefix[mid] <= lt) lo = mid; else hi = mid - 1;
    }
    g = lo;
    local = lt - p.prefix[g];
  }

  const TE *A, *B, *B2;
  TE *C;
  long lda, ldb, ldc;           // row strides
  size_t akc = BKE, bkc = BKE;  // k-chunk strides
  int M, N, K;
  int r0;
  const int32_t *gat = nullptr;  // routed rows gathered from the expert input
  int slot = -1;                 // EPI_PIECE: float32 partial slot of a cut window, or -1
  if (p.kwin) {
    int grp = g, k0, k1;
    if (p.pieces) {
      const int32_t *pc = p.pieces + 4 * (size_t)g;
      grp = pc[0]; k0 = pc[1]; k1 = pc[2]; slot = pc[3];
    } else {
      k0 = p.kwin[g]; k1 = p.kwin[g + 1];
    }
    r0 = 0;
    M = p.Mk; N = p.N; K = k1 - k0;
    lda = BKE; ldb = BKE; ldc = p.ldc;
    akc = (size_t)p.lda * BKE; bkc = (size_t)p.ldb * BKE;
    A = (const TE *)p.A + (size_t)(k0 / BKE) * akc;
    B = (const TE *)p.B + (size_t)(k0 / BKE) * bkc;
    B2 = nullptr;
    C = (TE *)p.C + (size_t)grp * p.cstride;
  } else if (g < p.E) {
    r0 = p.offsets[g];
    M = p.offsets[g + 1] - r0;
    lda = p.lda; ldb = p.ldb; ldc = p.ldc; N = p.N; K = p.K;
    A = (const TE *)p.A;
    if (p.gather) {
      gat = p.gather;
      A += (size_t)(g / p.gEh) * p.gdh;
    }
    B = (const TE *)p.B + (size_t)g * p.bstride;
    B2 = p.B2 ? (const TE *)p.B2 + (size_t)g * p.bstride : nullptr;
    C = (TE *)p.C;
  } else {
    r0 = 0;
    M = p.Mx; N = p.Nx; K = p.Kx;
    lda = p.ldax; ldb = p.ldbx; ldc = p.ldcx;
    A = (const TE *)p.Ax; B = (const TE *)p.Bx; B2 = (const TE *)p.Bx2; C = (TE *)p.Cx;
  }
  int wbeg;
  row_window(p.split, M, &wbeg, &M);
  r0 += wbeg;
  if (!gat) A += (size_t)r0 * lda;
  C += (size_t)r0 * ldc;
  // grouped raster inside the group: bands of GM m-tiles, n outer, m inner
  const int mt = (M + BM_ - 1) / BM_, nt = n_tiles<EPI, BN_>(N);
  constexpr int GM = 8;
  const int band = local / (GM * nt);
  const int first_m = band * GM;
  const int gsm = min(mt - first_m, GM);
  const int in_band = local - band * GM * nt;
  const int tm = first_m + in_band % gsm;
  const int tn = in_band / gsm;
  const int m0 = tm * BM_;
  constexpr int HB = BN_ / 2;  // SwiGLU: hidden columns per tile

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wm = wv / WGN, wn = wv % WGN;
  const int cq = lane >> 4, l16 = lane & 15;

  // global source of each LDS slot s = i*NT + tid this thread fills, as a
  // 32-bit element offset from the operand base (a group's operand is < 2^31
  // elements); SwiGLU B rows past HB come from the up projection
  uint32_t oa[LA], ob[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int s = i * NT + tid, row = s / KS, q = swz<KS>(row, s % KS);
    const int ar = min(m0 + row, M - 1);
    const size_t arow = gat ? (size_t)(gat[r0 + ar] / p.gK) : (size_t)ar;
    oa[i] = (uint32_t)(arow * lda + q * EPC);
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int s = i * NT + tid, row = s / KS, q = swz<KS>(row, s % KS);
    if (kPair<EPI>) {
      const int hn = min(tn * HB + (row % HB), N - 1);
      ob[i] = (uint32_t)((size_t)hn * ldb + q * EPC);
    } else {
      ob[i] = (uint32_t)((size_t)min(tn * BN_ + row, N - 1) * ldb + q * EPC);
    }
  }
  auto bsrc = [&](int i) -> const TE * {  // which projection slot i reads
    const int row = (i * NT + tid) / KS;
    return (kPair<EPI> && row >= HB) ? B2 : B;
  };
  const int nk = K / BKE;
  f32x4 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS slot of this lane's fragments: fragment rows are multiples of 16 plus
  // l16, so row & 7 == l16 & 7 and the swizzled slot depends only on the
  // k-step; the per-fragment part is a compile-time offset
  static_assert(KS == 8, "fragment addressing assumes 128-byte k-chunks");
  int abase[NKS], bbase[NKS];
  const int bwoff = kPair<EPI> ? wn * (HB / WGN) : wn * WN;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int sw = swz<KS>(l16, cq + 4 * ks);
    abase[ks] = (wm * WM + l16) * KS + sw;
    bbase[ks] = (bwoff + l16) * KS + sw;
  }
  auto brow_off = [](int f) {  // B-tile row of n-fragment f, relative to bwoff
    return kPair<EPI> ? ((f < NF / 2) ? f * 16 : HB + (f - NF / 2) * 16) : f * 16;
  };

  auto issue_a = [&](int kc, int st) {
    const size_t ko = (size_t)kc * akc;
#pragma unroll
    for (int i = 0; i < LA; ++i) load_lds16(A + oa[i] + ko, sA + st * SA + i * NT + wv * 64);
  };
  auto issue_b = [&](int kc, int st) {
    const size_t ko = (size_t)kc * bkc;
#pragma unroll
    for (int i = 0; i < LB; ++i) load_lds16(bsrc(i) + ob[i] + ko, sB + st * SB + i * NT + wv * 64);
  };
  // NL: m-fragments of this wave that hold rows (the rest of a ragged tile is
  // skipped: no LDS reads, no MFMAs)
  auto read = [&](auto nl, int sa, int sb, int ks, u32x4 *fa, u32x4 *fb) {
    constexpr int NL = decltype(nl)::value;
    if constexpr (NL > 0) {
#pragma unroll
      for (int i = 0; i < NL; ++i) fa[i] = sA[sa * SA + abase[ks] + i * 16 * KS];
#pragma unroll
      for (int f = 0; f < NF; ++f) fb[f] = sB[sb * SB + bbase[ks] + brow_off(f) * KS];
    }
  };
  auto mfma = [&](auto nl, const u32x4 *fa, const u32x4 *fb) {
    constexpr int NL = decltype(nl)::value;
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[i][f] = mma16(fb[f], fa[i], acc[i][f], TE());
  };
  // scheduling hint (SG): interleave the LDS reads of the next k-step with the
  // MFMAs of the current one
  auto interleave = [&](auto nl) {
    constexpr int NL = decltype(nl)::value;
    if constexpr (SG && NL > 0) {
      constexpr int NR = NL + NF, NM = NL * NF;
      constexpr int PER = NM / NR > 0 ? NM / NR : 1;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one DS read
        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // then PER MFMAs
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
    }
  };

  // Software pipeline.  Step kc (after its barrier) loads A chunk kc+STA into
  // the A stage of chunk kc and B chunk kc+STB into the B stage of chunk kc;
  // the LDS reads of each k-step overlap the MFMAs of the one before.  The
  // prologue issues the loads of the steps before step 0 in the same order.
  // Vector-memory loads complete in order, so "chunk c has landed" is a wait
  // until no more than the loads issued after it are outstanding:
  constexpr int SMAX = STA > STB ? STA : STB, SMIN = STA < STB ? STA : STB;
  constexpr int LAFTER = (STA < STB ? LB : 0) + (SMIN - 2) * (LA + LB);
  auto wait_chunk = [&](int c) {  // chunk c landed (all chunks < c + SMAX - 1 issued, if they exist)
    if (c + SMAX - 2 < nk) wait_vmcnt<LAFTER>(); else wait_vmcnt0();
  };
  auto pipeline = [&](auto nl) {
    u32x4 fa0[MF], fb0[NF], fa1[MF], fb1[NF];
    for (int i = -SMAX; i < 0; ++i) {
      if (i + STA >= 0 && i + STA < nk) issue_a(i + STA, i + STA);
      if (i + STB >= 0 && i + STB < nk) issue_b(i + STB, i + STB);
    }
    wait_chunk(0);
    barrier_nofence();
    read(nl, 0, 0, 0, fa0, fb0);
    int sa = 0, sb = 0;
    for (int kc = 0; kc < nk; ++kc) {
      read(nl, sa, sb, 1, fa1, fb1);
      mfma(nl, fa0, fb0);
      interleave(nl);
      const int san = (sa + 1 == STA) ? 0 : sa + 1, sbn = (sb + 1 == STB) ? 0 : sb + 1;
      if (kc + 1 < nk) {
        // chunk kc+1 landed for this wave; this wave's reads of chunk kc are done
        wait_chunk(kc + 1);
        wait_lgkmcnt0();
        barrier_nofence();
        if (kc + STA < nk) issue_a(kc + STA, sa);
        if (kc + STB < nk) issue_b(kc + STB, sb);
      }
      // on the last chunk this reads stage data that is never used
      read(nl, san, sbn, 0, fa0, fb0);
      mfma(nl, fa1, fb1);
      interleave(nl);
      sa = san;
      sb = sbn;
    }
  };
  // live m-fragments of this wave, rounded up to MF, MF/2, MF/4 or 0 (the
  // rows past M in a group's last tile); wave-uniform, so every wave still
  // takes part in the loads and barriers
  const int live = min(max(M - m0 - wave_id() / WGN * WM, 0), WM);
  if (live > WM / 2) pipeline(std::integral_constant<int, MF>{});
  else if (MF >= 4 && live > WM / 4) pipeline(std::integral_constant<int, (MF >= 4 ? MF / 2 : MF)>{});
  else if (live > 0) pipeline(std::integral_constant<int, (MF >= 4 ? MF / 4 : MF)>{});
  else pipeline(std::integral_constant<int, 0>{});

  // epilogue.  The MFMAs take the B fragment as their first operand, so they
  // produce C^T blocks: acc[i][f][v] = C[row wm*WM + i*16 + l16][column
  // (n-fragment f) + 4*cq + v], four consecutive columns of one row per lane,
  // written (and, for the residual, read) as one 8-byte (bf16) or 16-byte
  // (fp32) access.  Every N here is a multiple of 64, so a quad is either
  // wholly inside N or wholly outside.
  const TE *R = (EPI == EPI_RESID) ? (const TE *)p.res + (size_t)r0 * p.ldres : nullptr;
  const TE *DHp = (EPI == EPI_SWIGLU_BWD || EPI == EPI_RELU_BWD) ? (const TE *)p.dh + (size_t)r0 * p.lddh : nullptr;
  TE *HO = (EPI == EPI_SWIGLU_BWD || EPI == EPI_RELU_BWD) ? (TE *)p.hout + (size_t)r0 * p.ldh : nullptr;
  // the forward's pre-activations, kept for the backward when asked for
  TE *GS = ((EPI == EPI_SWIGLU || EPI == EPI_RELU) && p.gsave) ? (TE *)p.gsave + (size_t)r0 * p.ldg : nullptr;
  // The epilogues that read a second operand (the residual; the backward's
  // upstream dH) issue all of the wave's loads before its first store: C may
  // alias that operand as far as the compiler knows, so a load placed after a
  // store would wait for it, and the load latencies would add up tile by tile.
  constexpr bool kRd = EPI == EPI_RESID || EPI == EPI_SWIGLU_BWD || EPI == EPI_RELU_BWD;
  constexpr int NQ = kPair<EPI> ? NF / 2 : NF;  // quads per fragment row that the epilogue reads
  auto qcol = [&](int f) {
    return kPair<EPI> ? tn * HB + wn * (HB / WGN) + f * 16 + 4 * cq : tn * BN_ + wn * WN + f * 16 + 4 * cq;
  };
  typename Quad<TE>::Raw pre[kRd ? MF : 1][kRd ? NQ : 1];
  // The residual (bf16, when the stages hold a whole tile of it) comes in
  // through LDS: whole rows in coalesced 16-byte direct loads, into slots
  // XOR-swizzled by row (slot q of row r at r * QR + (q ^ r % QR)) so that
  // the 16 rows one quad read touches fall in distinct banks.  Read straight
  // from global memory, each wave load instruction would touch 16 rows for 32
  // bytes of each.
  constexpr int RQR = BN_ * (int)sizeof(TE) / 16;  // 16-byte slots per residual row
  constexpr bool kResLds = EPI == EPI_RESID && sizeof(TE) == 2 && BM_ * RQR <= STA * SA + STB * SB &&
                           (RQR & (RQR - 1)) == 0;
  if constexpr (kResLds) {
    // every wave's LDS reads of the last chunk are done before the stages are overwritten
    wait_lgkmcnt0();
    barrier_nofence();
    const int cmax = N - tn * BN_;  // columns of this tile inside N (a multiple of 64)
#pragma unroll 4
    for (int s0 = 0; s0 < BM_ * RQR; s0 += NT) {
      const int sl = s0 + tid, r = sl / RQR, q = (sl % RQR) ^ (r % RQR);
      // rows past M and columns past N read the tile's first element (never used)
      const bool in = m0 + r < M && q * 8 < cmax;
      load_lds16(R + (in ? (size_t)(m0 + r) * p.ldres + tn * BN_ + q * 8 : (size_t)m0 * p.ldres + tn * BN_),
                 smem + s0 + wv * 64);
    }
    wait_vmcnt0();
    barrier_nofence();
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int rt = wm * WM + i * 16 + l16;
#pragma unroll
      for (int f = 0; f < NQ; ++f) {
        const int ct = qcol(f) - tn * BN_, q = ct / 8;
        const char *src = (const char *)(smem + rt * RQR + (q ^ (rt % RQR))) + (ct % 8) * 2;
        pre[i][f] = *(const typename Quad<TE>::Raw *)src;
      }
    }
  } else if constexpr (kRd) {
    const TE *src = (EPI == EPI_RESID) ? R : DHp;
    const long lds = (EPI == EPI_RESID) ? p.ldres : p.lddh;
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int row = m0 + wm * WM + i * 16 + l16;
#pragma unroll
      for (int f = 0; f < NQ; ++f) {
        const int col = qcol(f);
        pre[i][f] = (row < M && col < N) ? Quad<TE>::raw(src + (size_t)row * lds + col) : typename Quad<TE>::Raw{};
      }
    }
  }
  // The plain, ReLU and residual epilogues (bf16) hand their output tile to
  // the global stores through LDS as well: each wave writes its quads into
  // the swizzled slots, then every thread stores whole 16-byte slots of
  // whole rows.
  constexpr bool kStageC = (EPI == EPI_PLAIN || EPI == EPI_RELU || EPI == EPI_RESID) && sizeof(TE) == 2 &&
                           BM_ * RQR <= STA * SA + STB * SB && (RQR & (RQR - 1)) == 0;
  if constexpr (kStageC) {
    // every wave's LDS reads (last chunk, staged residual) are done
    wait_lgkmcnt0();
    barrier_nofence();
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int rt = wm * WM + i * 16 + l16;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int ct = wn * WN + f * 16 + 4 * cq;
        float o[4], r[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (EPI == EPI_RESID) Quad<TE>::decode(pre[i][f], r);
        if constexpr (EPI == EPI_RELU) {
          if (GS && m0 + rt < M && tn * BN_ + ct < N) {
            const float a[4] = {acc[i][f][0], acc[i][f][1], acc[i][f][2], acc[i][f][3]};
            Quad<TE>::store(GS + (size_t)(m0 + rt) * p.ldg + tn * BN_ + ct, a);
          }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          o[v] = acc[i][f][v];
          if (EPI == EPI_RELU) o[v] = fmaxf(o[v], 0.0f);
          if (EPI == EPI_RESID) o[v] += r[v];
        }
        Quad<TE>::store((TE *)((char *)(smem + rt * RQR + ((ct / 8) ^ (rt % RQR))) + (ct % 8) * 2), o);
      }
    }
    wait_lgkmcnt0();
    barrier_nofence();
    const int cmax = N - tn * BN_;
#pragma unroll 4
    for (int s0 = 0; s0 < BM_ * RQR; s0 += NT) {
      const int sl = s0 + tid, r = sl / RQR, q = (sl % RQR) ^ (r % RQR);
      if (m0 + r < M && q * 8 < cmax) *(u32x4 *)(C + (size_t)(m0 + r) * ldc + tn * BN_ + q * 8) = smem[sl];
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int row = m0 + wm * WM + i * 16 + l16;
    if (row >= M) continue;
    if (EPI == EPI_SWIGLU_BWD) {
      // recomputed gate g and up u with the upstream dH: dA = dH * u * SiLU'(g),
      // dB = dH * SiLU(g) (C[row][col] and C[row][N + col]), H = SiLU(g) * u
#pragma unroll
      for (int f = 0; f < NF / 2; ++f) {
        const int col = qcol(f);
        if (col >= N) continue;
        float dh[4], da[4], db[4], h[4];
        Quad<TE>::decode(pre[i][f], dh);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gt = acc[i][f][v], up = acc[i][f + NF / 2][v];
          const float sg = 1.0f / (1.0f + __expf(-gt)), si = gt * sg;
          da[v] = dh[v] * up * (sg * (1.0f + gt * (1.0f - sg)));
          db[v] = dh[v] * si;
          h[v] = si * up;
        }
        Quad<TE>::store(C + (size_t)row * ldc + col, da);
        Quad<TE>::store(C + (size_t)row * ldc + N + col, db);
        Quad<TE>::store(HO + (size_t)row * p.ldh + col, h);
      }
    } else if (EPI == EPI_RELU_BWD) {
      // recomputed a = W1 v with the upstream dH: dA = dH * [a > 0], H = max(a, 0)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int col = qcol(f);
        if (col >= N) continue;
        float dh[4], da[4], h[4];
        Quad<TE>::decode(pre[i][f], dh);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float a = acc[i][f][v];
          da[v] = a > 0.0f ? dh[v] : 0.0f;
          h[v] = fmaxf(a, 0.0f);
        }
        Quad<TE>::store(C + (size_t)row * ldc + col, da);
        Quad<TE>::store(HO + (size_t)row * p.ldh + col, h);
      }
    } else if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int f = 0; f < NF / 2; ++f) {
        const int col = tn * HB + wn * (HB / WGN) + f * 16 + 4 * cq;
        if (col >= N) continue;
        float h[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gt = acc[i][f][v], up = acc[i][f + NF / 2][v];
          h[v] = gt / (1.0f + __expf(-gt)) * up;
        }
        Quad<TE>::store(C + (size_t)row * ldc + col, h);
        if (GS) {
          const float gq[4] = {acc[i][f][0], acc[i][f][1], acc[i][f][2], acc[i][f][3]};
          const float uq[4] = {acc[i][f + NF / 2][0], acc[i][f + NF / 2][1], acc[i][f + NF / 2][2],
                               acc[i][f + NF / 2][3]};
          Quad<TE>::store(GS + (size_t)row * p.ldg + col, gq);
          Quad<TE>::store(GS + (size_t)row * p.ldg + N + col, uq);
        }
      }
    } else if (EPI == EPI_PIECE) {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int col = tn * BN_ + wn * WN + f * 16 + 4 * cq;
        if (col >= N) continue;
        if (slot >= 0) {
          *(float4 *)(p.part + (size_t)slot * M * N + (size_t)row * N + col) =
              make_float4(acc[i][f][0], acc[i][f][1], acc[i][f][2], acc[i][f][3]);
        } else {
          const float o[4] = {acc[i][f][0], acc[i][f][1], acc[i][f][2], acc[i][f][3]};
          Quad<TE>::store(C + (size_t)row * ldc + col, o);
        }
      }
    } else if (EPI == EPI_F32OUT) {
      float *Cf = (float *)p.C + (size_t)g * p.cstride + (size_t)r0 * ldc;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int col = tn * BN_ + wn * WN + f * 16 + 4 * cq;
        if (col >= N) continue;
        *(float4 *)(Cf + (size_t)row * ldc + col) =
            make_float4(acc[i][f][0], acc[i][f][1], acc[i][f][2], acc[i][f][3]);
      }
    } else {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int col = tn * BN_ + wn * WN + f * 16 + 4 * cq;
        if (col >= N) continue;
        float o[4], r[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (EPI == EPI_RESID) Quad<TE>::decode(pre[i][f], r);
        if constexpr (EPI == EPI_RELU) {
          if (GS) {
            const float a[4] = {acc[i][f][0], acc[i][f][1], acc[i][f][2], acc[i][f][3]};
            Quad<TE>::store(GS + (size_t)row * p.ldg + col, a);
          }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          o[v] = acc[i][f][v];
          if (EPI == EPI_RELU) o[v] = fmaxf(o[v], 0.0f);
          if (EPI == EPI_RESID) o[v] += r[v];
        }
        Quad<TE>::store(C + (size_t)row * ldc + col, o);
      }
    }
  }
}

// ---------------------------------------------------------------- host
// Tile shapes with an instantiated kernel.
enum TileCfg {
  TILE_128x128 = 0,     // 4 waves (2 x 2), wave tile 64 x 64 (also the float32 tile)
  TILE_256x256_W8 = 1,  // 8 waves (2 x 4), wave tile 128 x 64; head + tail launches
  TILE_128x128_W8 = 2,  // 8 waves (2 x 4), wave tile 64 x 32
  TILE_MIXED = 3,       // routed groups of very unequal size: 256-row tiles for the large, 128 for the rest
  TILE_TAIL = 4,        // 8 waves (4 x 2), wave tile 32 x 32, deep rings: the short tails of 256-row launches
};
// The tail launch of a 256-row product holds at most 128 rows per group, so
// each of its tiles streams a weight column tile once for few rows.  When
// its 128 x 128 tiles are too few to give every CU two (a narrow, deep
// product: the down projection, d_model columns over d_ff), it runs 128 x 64
// tiles instead, twice the blocks, with the weight chunks kTailStagesB deep:
// measured on the coarse 8-expert layer, that tail launch 160 -> 108 us.  A
// wide product keeps the 128-wide tile (its 64-wide tiles would read every
// row chunk twice as often: gate/up tail 174 -> 205 us).
constexpr int kTailStagesA = 3, kTailStagesB = 8;

static long max_tiles(long rows_bound, int groups, int bm, int ntiles) {
  return ((rows_bound + bm - 1) / bm + groups) * ntiles;
}

// The kernel launch of one tile shape.  a.prefix: the device tile prefix
// (routed groups), or NULL with a.fixed_tiles set (a plain product).
template <typename TE, int EPI, int BM_, int BN_, int WGM, int WGN, int KS, int STA, int STB, bool SG = false>
static int run_gemm_t(GemmArgs a, hipStream_t st) {
  // grid: an upper bound of the tile count; blocks past the device-built
  // prefix total exit at once.  A tail launch holds at most one tile row per
  // group.
  long grid;
  if (!a.prefix)
    grid = a.fixed_tiles;
  else if (a.split == 2)
    grid = (long)a.E * n_tiles<EPI, BN_>(a.N) + (a.has_x ? n_tiles<EPI, BN_>(a.Nx) : 0);
  else
    grid = (a.E ? max_tiles(a.Mr_bound, a.E, BM_, n_tiles<EPI, BN_>(a.N)) : 0) +
           (a.has_x ? max_tiles(a.Mx, 0, BM_, n_tiles<EPI, BN_>(a.Nx)) : 0);
  // the large groups' launch of a mixed pair: its windows are whole 256-row
  // tiles, so at most Mr_bound / 256 tile rows (blocks past the prefix total,
  // all of them when no group is large, exit at once)
  if (a.split == 3) grid = (a.Mr_bound / BM_) * n_tiles<EPI, BN_>(a.N);
  if (grid <= 0) return 0;
  // dynamic LDS up to the device's per-workgroup limit (160 KiB on gfx950)
  constexpr size_t lds = (size_t)(STA * BM_ + STB * BN_) * KS * 16;
  static_assert(lds <= 160 * 1024, "LDS per workgroup");
  hipLaunchKernelGGL((grouped_gemm_kernel<TE, EPI, BM_, BN_, WGM, WGN, KS, STA, STB, SG>), dim3(grid),
                     dim3(64 * WGM * WGN), lds, st, a);
  return launch_status("grouped gemm");
}

template <typename TE, int EPI>
static int run_gemm_one(GemmArgs a, int tile, hipStream_t st) {
  if constexpr (sizeof(TE) == 4) {
    return run_gemm_t<TE, EPI, 128, 128, 2, 2, 8, 2, 2>(a, st);
  } else {
    switch (tile) {
      case TILE_256x256_W8: return run_gemm_t<TE, EPI, 256, 256, 2, 4, 8, 2, 2, true>(a, st);
      case TILE_128x128_W8:
        // the down projection (long K, few row tiles per weight tile) keeps a
        // third weight chunk in flight; measured: -27 % on a tail launch of
        // a few short groups, -6 % on 160 experts of ~280 rows; no gain for
        // the gate/up launch, which streams at HBM rate
        if constexpr (EPI == EPI_PLAIN || EPI == EPI_RESID)
          return run_gemm_t<TE, EPI, 128, 128, 2, 4, 8, 2, 3, true>(a, st);
        else
          return run_gemm_t<TE, EPI, 128, 128, 2, 4, 8, 2, 2, true>(a, st);
      case TILE_TAIL: return run_gemm_t<TE, EPI, 128, 64, 4, 2, 8, kTailStagesA, kTailStagesB, true>(a, st);
      default: return run_gemm_t<TE, EPI, 128, 128, 2, 2, 8, 2, 2>(a, st);
    }
  }
}

// One launch of a product: its tile shape and row window.  256-row tiles run
// as a head launch (split 1) plus a tail launch (split 2) of 128-row tiles,
// 64 columns wide when the groups' 128 x 128 tail tiles would not give every
// CU two (groups: the groups of the product, N its output columns).
struct Launch {
  int tile, split;
};
static int col_tiles(int epi, int tile, int N);
static int plan_launches(int tile, int epi, int N, int groups, Launch out[2]) {
  if (tile == TILE_256x256_W8) {
    out[0] = {TILE_256x256_W8, 1};
    out[1] = {(long)groups * col_tiles(epi, TILE_128x128_W8, N) < 2 * 256 ? TILE_TAIL : TILE_128x128_W8, 2};
    return 2;
  }
  if (tile == TILE_MIXED) {
    out[0] = {TILE_256x256_W8, 3};
    out[1] = {TILE_128x128_W8, 4};
    return 2;
  }
  out[0] = {tile, 0};
  return 1;
}
static int tile_rows(int tile) { return tile == TILE_256x256_W8 ? 256 : 128; }
static int tile_cols(int tile) { return tile == TILE_256x256_W8 ? 256 : tile == TILE_TAIL ? 64 : 128; }
static int col_tiles(int epi, int tile, int N) {
  const int bn = tile_cols(tile);
  return (epi == EPI_SWIGLU || epi == EPI_SWIGLU_BWD) ? (N + bn / 2 - 1) / (bn / 2) : (N + bn - 1) / bn;
}
static PrepCfg prep_cfg(int epi, const Launch &l, int N, int Nx) {
  return PrepCfg{tile_rows(l.tile), l.split, col_tiles(epi, l.tile, N), col_tiles(epi, l.tile, Nx)};
}

// tile shape for a product: large tiles when the groups are tall enough to fill them
static int pick_tile(long rows, int groups) {
  long avg = groups > 0 ? rows / groups : rows;
  return avg >= 1024 ? TILE_256x256_W8 : TILE_128x128_W8;
}

// Routed products.  With expert choice every expert holds exactly min(C, T)
// rows (known here): the big tile unless its last row tile would be mostly
// padding.  Otherwise only the average and the largest possible group are
// known here (the rows per expert are on the device): tall groups on average
// take the big tile; short ones the small tile, in a mixed pair when a group
// can reach SPLIT_HOT rows (no capacity, or a capacity that large), so that
// hot experts still get the big tile.
static int pick_tile_routed(const Shape &s) {
  if (s.expert_choice) {
    const long n = std::min<long>(s.C, s.T);
    const long waste = (n + 255) / 256 * 256 - n;
    return (n >= 256 && waste * 8 <= n) ? TILE_256x256_W8 : TILE_128x128_W8;
  }
  const int t = pick_tile(s.R_max, s.E);
  const long most = s.drop == DROP_CAPACITY ? std::min<long>(s.C, s.T) : s.T;  // rows one expert can hold
  return (t == TILE_128x128_W8 && most >= SPLIT_HOT) ? TILE_MIXED : t;
}

// A plain product (one group, no routed rows: a.E == 0, a.has_x == 1): the
// tile count of each launch is known on the host; launches with no tiles are
// skipped.
template <typename TE, int EPI>
static int run_plain(GemmArgs a, int tile, hipStream_t st) {
  Launch l[2];
  const int nl = plan_launches(tile, EPI, a.Nx, 1, l);
  for (int i = 0; i < nl; ++i) {
    int beg, len;
    row_window(l[i].split, a.Mx, &beg, &len);
    a.split = l[i].split;
    a.prefix = nullptr;
    a.fixed_tiles = (len + tile_rows(l[i].tile) - 1) / tile_rows(l[i].tile) * col_tiles(EPI, l[i].tile, a.Nx);
    if (a.fixed_tiles == 0) continue;
    if (int rc = run_gemm_one<TE, EPI>(a, l[i].tile, st)) return rc;
  }
  return 0;
}

// ---------------------------------------------------------------- backward products
template <typename TE>
static int run_epi(int epi, const GemmArgs &a, int tile, hipStream_t st) {
  switch (epi) {
    case EPI_PLAIN: return run_gemm_one<TE, EPI_PLAIN>(a, tile, st);
    case EPI_SWIGLU_BWD: return run_gemm_one<TE, EPI_SWIGLU_BWD>(a, tile, st);
    case EPI_RELU_BWD: return run_gemm_one<TE, EPI_RELU_BWD>(a, tile, st);
    case EPI_F32OUT:
      if constexpr (sizeof(TE) == 2) return run_gemm_one<TE, EPI_F32OUT>(a, tile, st);
      else return run_gemm_one<TE, EPI_PLAIN>(a, tile, st);  // float32 output already
    default: return -2;
  }
}

// C[R, N] = A[R, K] B_e[N, K]^T over the rows of every routed expert e
// (A rows gathered from the expert input when `gather`), epilogue `epi`
int gemm_routed(const Shape &s, int epi, const void *A, long lda, const int32_t *gather, const void *B,
                const void *B2, long ldb, long bstride, void *C, long ldc, int N, int K, const int32_t *offsets,
                const void *dh, long lddh, void *hout, long ldh, int32_t *prefix, hipStream_t st) {
  GemmArgs a{};
  a.A = A; a.lda = lda; a.gather = gather; a.gK = s.K; a.gEh = s.Eh; a.gdh = s.dh;
  a.B = B; a.B2 = B2; a.ldb = ldb; a.bstride = bstride; a.C = C; a.ldc = ldc;
  a.offsets = offsets; a.E = s.E; a.N = N; a.K = K; a.Mr_bound = s.R_max; a.G = s.E;
  a.dh = dh; a.lddh = lddh; a.hout = hout; a.ldh = ldh;
  const int tile = s.act_f32 ? TILE_128x128 : pick_tile_routed(s);
  Launch l[2];
  const int nl = plan_launches(tile, epi, N, s.E, l);
  PrepArgs pa{};
  pa.offsets = offsets; pa.E = s.E; pa.has_x = 0; pa.Mx = 0; pa.prefix = prefix;
  for (int i = 0; i < nl; ++i) pa.c[i] = prep_cfg(epi, l[i], N, 0);
  hipLaunchKernelGGL(gemm_prep_kernel, dim3(nl), dim3(1024), 0, st, pa);
  if (int rc = launch_status("gemm tile prefix")) return rc;
  for (int i = 0; i < nl; ++i) {
    a.split = l[i].split;
    a.prefix = prefix + (size_t)i * (s.E + 2);
    const int rc = s.act_f32 ? run_epi<float>(epi, a, l[i].tile, st) : run_epi<uint16_t>(epi, a, l[i].tile, st);
    if (rc) return rc;
  }
  return 0;
}

// C[M, N] = A[M, K] B[N, K]^T, one plain group
int gemm_plain(bool f32, int epi, const void *A, long lda, const void *B, const void *B2, long ldb, void *C,
               long ldc, int M, int N, int K, const void *dh, long lddh, void *hout, long ldh, hipStream_t st) {
  GemmArgs a{};
  a.E = 0; a.has_x = 1; a.G = 1;
  a.Ax = A; a.ldax = lda; a.Bx = B; a.Bx2 = B2; a.ldbx = ldb; a.Cx = C; a.ldcx = ldc; a.Mx = M; a.Nx = N; a.Kx = K;
  a.dh = dh; a.lddh = lddh; a.hout = hout; a.ldh = ldh;
  const int tile = f32 ? TILE_128x128 : pick_tile(M, 1);
  Launch l[2];
  const int nl = plan_launches(tile, epi, N, 1, l);
  for (int i = 0; i < nl; ++i) {
    int beg, len;
    row_window(l[i].split, M, &beg, &len);
    a.split = l[i].split;
    a.prefix = nullptr;
    a.fixed_tiles = (len + tile_rows(l[i].tile) - 1) / tile_rows(l[i].tile) * col_tiles(epi, l[i].tile, N);
    if (a.fixed_tiles == 0) continue;
    const int rc = f32 ? run_epi<float>(epi, a, l[i].tile, st) : run_epi<uint16_t>(epi, a, l[i].tile, st);
    if (rc) return rc;
  }
  return 0;
}

// One group's C[M, N] = A[:, 0..Kt) B[:, 0..Kt)^T, A and B k-chunked with lda and
// ldb rows, K split into `nsplit` windows kwin[0..nsplit] (device, multiples
// of 64): each window's product
// goes to part[s] (float32, M x N, row stride N), then C = sum over s in
// order, rounded once.  Fills the chip when one group has few output tiles.
// c[0..3] = sum over s < nsplit of p[s * stride + 0..3], in order s = 0, 1, ...,
// rounded once; up to eight partials' loads in flight before their adds
template <typename TE>
__device__ __forceinline__ void reduce_quad(const float *__restrict__ p, size_t stride, int nsplit,
                                            TE *__restrict__ c) {
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < nsplit) v[u] = *(const float4 *)(p + (size_t)(s0 + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < nsplit) {
        o[0] += v[u].x; o[1] += v[u].y; o[2] += v[u].z; o[3] += v[u].w;
      }
  }
  Quad<TE>::store(c, o);
}

// C = sum of the partials in order (n a multiple of 4: four columns per thread)
template <typename TE>
__global__ void splitk_reduce_kernel(const float *__restrict__ part, long n, int nsplit, TE *__restrict__ C) {
  for (long i = 4 * (blockIdx.x * (long)blockDim.x + threadIdx.x); i < n; i += 4L * gridDim.x * blockDim.x)
    reduce_quad(part + i, (size_t)n, nsplit, C + i);
}

int gemm_splitk(bool f32, const void *A, long lda, const void *B, long ldb, void *C, int M, int N, int nsplit,
                const int32_t *kwin, float *part, hipStream_t st) {
  if (M <= 0 || N <= 0 || nsplit <= 0) return 0;
  GemmArgs a{};
  a.A = A; a.lda = lda; a.B = B; a.ldb = ldb; a.C = part; a.ldc = N; a.cstride = (long)M * N;
  a.kwin = kwin; a.Mk = M; a.N = N; a.E = nsplit; a.G = nsplit; a.split = 0; a.prefix = nullptr;
  const int tile = f32 ? TILE_128x128 : (M >= 256 && N >= 256 ? TILE_256x256_W8 : TILE_128x128_W8);
  a.fixed_tiles = nsplit * ((M + tile_rows(tile) - 1) / tile_rows(tile)) * col_tiles(EPI_PLAIN, tile, N);
  const int rc = f32 ? run_gemm_one<float, EPI_PLAIN>(a, tile, st) : run_gemm_one<uint16_t, EPI_F32OUT>(a, tile, st);
  if (rc) return rc;
  const long n = (long)M * N;  // N is a multiple of 64
  const unsigned grid = (unsigned)std::min<long>((n / 4 + 255) / 256, 8192);
  if (f32)
    hipLaunchKernelGGL((splitk_reduce_kernel<float>), dim3(grid), dim3(256), 0, st, part, n, nsplit, (float *)C);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<uint16_t>), dim3(grid), dim3(256), 0, st, part, n, nsplit,
                       (uint16_t *)C);
  return launch_status("split-k reduce");
}

// ---------------------------------------------------------------- K-grouped pieces
// The per-expert windows cut in pieces of at most `depth` columns each
// (multiples of 64, near-equal within an expert): expert e's window of n_e
// columns gives P_e = max(1, ceil(n_e / depth)) pieces.  A whole window (P_e
// == 1) writes its product straight to C_e; the pieces of a cut window write
// float32 partials to consecutive slots (in expert, then piece order), added
// afterwards in order.  The table lists the pieces deepest first, so the
// tiles dispatched first are the longest (the hardware hands blocks to free
// CUs in order: longest-first list scheduling); the order of equal depths is
// free, and no result depends on it.  One block of 1024 threads: tab[p] =
// (e, k0, k1, slot), tab[4 * maxp] = P (maxp bounds P), and for the
// reduction red[e] = (first slot, P_e or 0 when whole).
constexpr int PIECE_BUCKETS = 2048;  // depth classes (64-column chunks; deeper pieces share the last)
__global__ __launch_bounds__(1024) void kgroup_pieces_kernel(const int32_t *__restrict__ kwin, int G, int depth,
                                                             long maxp, int32_t *__restrict__ tab,
                                                             int32_t *__restrict__ red) {
  __shared__ int sp[1024], ss[1024], hist[PIECE_BUCKETS];
  const int tid = threadIdx.x, per = (G + 1023) / 1024;
  for (int b = tid; b < PIECE_BUCKETS; b += 1024) hist[b] = 0;
  int np[8], ns[8], sum_p = 0, sum_s = 0;
  // bucket of a piece: deepest first
  auto bucket = [](int chunks) { return PIECE_BUCKETS - 1 - min(chunks, PIECE_BUCKETS - 1); };
  __syncthreads();
  for (int i = 0; i < per && i < 8; ++i) {
    const int e = tid * per + i;
    int pe = 0;
    if (e < G) {
      const int n = kwin[e + 1] - kwin[e], chunks = n / 64;
      pe = n > depth ? (n + depth - 1) / depth : 1;
      for (int j = 0; j < pe; ++j)
        atomicAdd(&hist[bucket((int)((long)chunks * (j + 1) / pe) - (int)((long)chunks * j / pe))], 1);
    }
    np[i] = pe;
    ns[i] = pe > 1 ? pe : 0;
    sum_p += pe;
    sum_s += ns[i];
  }
  sp[tid] = sum_p;
  ss[tid] = sum_s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int up = tid >= o ? sp[tid - o] : 0, us = tid >= o ? ss[tid - o] : 0;
    __syncthreads();
    sp[tid] += up;
    ss[tid] += us;
    __syncthreads();
  }
  const int total = sp[1023];
  int rs = ss[tid] - sum_s;
  // exclusive prefix over the buckets (two per thread): a bucket's first position
  constexpr int BPT = PIECE_BUCKETS / 1024;
  static_assert(BPT * 1024 == PIECE_BUCKETS, "buckets per thread");
  int hb[BPT], hs = 0;
#pragma unroll
  for (int u = 0; u < BPT; ++u) { hb[u] = hist[tid * BPT + u]; hs += hb[u]; }
  __syncthreads();
  sp[tid] = hs;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int up = tid >= o ? sp[tid - o] : 0;
    __syncthreads();
    sp[tid] += up;
    __syncthreads();
  }
  int run = sp[tid] - hs;
#pragma unroll
  for (int u = 0; u < BPT; ++u) { hist[tid * BPT + u] = run; run += hb[u]; }
  __syncthreads();
  for (int i = 0; i < per && i < 8; ++i) {
    const int e = tid * per + i;
    if (e < G) {
      const int lo = kwin[e], chunks = (kwin[e + 1] - lo) / 64, pe = np[i];
      for (int j = 0; j < pe; ++j) {
        const int c0 = (int)((long)chunks * j / pe), c1 = (int)((long)chunks * (j + 1) / pe);
        int32_t *t = tab + 4 * (size_t)atomicAdd(&hist[bucket(c1 - c0)], 1);
        t[0] = e;
        t[1] = lo + c0 * 64;
        t[2] = lo + c1 * 64;
        t[3] = pe > 1 ? rs + j : -1;
      }
      red[2 * e] = rs;
      red[2 * e + 1] = pe > 1 ? pe : 0;
    }
    rs += ns[i];
  }
  if (tid == 0) tab[4 * maxp] = total;
}

// C_e = sum over its pieces' partials in order, rounded once (cut experts only);
// group e = blockIdx.y, four columns per thread (MN a multiple of 4)
template <typename TE>
__global__ void piece_reduce_kernel(const float *__restrict__ part, long MN, const int32_t *__restrict__ red,
                                    long cstride, TE *__restrict__ C) {
  const long e = blockIdx.y;
  const int first = red[2 * e], n = red[2 * e + 1];
  if (n == 0) return;
  const float *pe = part + (size_t)first * MN;
  for (long j = 4 * (blockIdx.x * (long)blockDim.x + threadIdx.x); j < MN; j += 4L * gridDim.x * blockDim.x)
    reduce_quad(pe + j, (size_t)MN, n, C + (size_t)e * cstride + j);
}

static int kgroup_tile(bool f32, int M, int N) {
  return f32 ? TILE_128x128 : (M >= 256 && N >= 256 ? TILE_256x256_W8 : TILE_128x128_W8);
}

// Piece depth for G groups of M x N outputs over at most Rp padded columns:
// the total depth over as many pieces as one round of resident tiles holds
// (at least 512 columns).  Windows of an even routing stay whole; a hot
// expert's window is cut into pieces no deeper than that.  (Finer pieces
// balance better but each cut piece writes and reads back an M x N float32
// partial; one round measured fastest on the skewed 64-expert workload.)
int kgroup_piece_depth(bool f32, int G, int M, int N, long Rp) {
  const int tile = kgroup_tile(f32, M, N);
  const long tpg = (long)((M + tile_rows(tile) - 1) / tile_rows(tile)) * col_tiles(EPI_PLAIN, tile, N);
  const long want = std::max<long>(1, ((tile == TILE_256x256_W8 ? 256 : 512) + tpg - 1) / tpg);
  const long d = (Rp + want - 1) / want;
  return (int)std::max<long>(512, (d + 63) / 64 * 64);
}
// bounds: pieces <= G + Rp / depth; partial slots (pieces of cut windows,
// each window deeper than depth) <= 2 * Rp / depth
long kgroup_max_pieces(int G, long Rp, int depth) { return G + Rp / depth + 1; }
long kgroup_max_slots(long Rp, int depth) { return 2 * Rp / depth + 1; }

int gemm_kgrouped_pieces(bool f32, const void *A, long lda, const void *B, long ldb, void *C, long ldc, long cstride,
                         int G, int M, int N, const int32_t *kwin, int depth, long max_pieces, int32_t *tab,
                         int32_t *red, float *part, hipStream_t st) {
  if (G <= 0 || M <= 0 || N <= 0) return 0;
  hipLaunchKernelGGL(kgroup_pieces_kernel, dim3(1), dim3(1024), 0, st, kwin, G, depth, max_pieces, tab, red);
  if (int rc = launch_status("weight-gradient pieces")) return rc;
  GemmArgs a{};
  a.A = A; a.lda = lda; a.B = B; a.ldb = ldb; a.C = C; a.ldc = ldc; a.cstride = cstride;
  a.kwin = kwin; a.Mk = M; a.N = N; a.E = G; a.G = G; a.split = 0; a.prefix = nullptr;
  a.pieces = tab; a.npieces = tab + 4 * max_pieces; a.part = part;
  const int tile = kgroup_tile(f32, M, N);
  a.fixed_tiles = (int)(max_pieces * ((M + tile_rows(tile) - 1) / tile_rows(tile)) * col_tiles(EPI_PLAIN, tile, N));
  const int rc = f32 ? run_gemm_one<float, EPI_PIECE>(a, tile, st) : run_gemm_one<uint16_t, EPI_PIECE>(a, tile, st);
  if (rc) return rc;
  const long mn = (long)M * N;  // N is a multiple of 64
  const dim3 grid((unsigned)std::min<long>((mn / 4 + 255) / 256, std::max<long>(1, 8192 / G)), (unsigned)G);
  if (f32)
    hipLaunchKernelGGL((piece_reduce_kernel<float>), grid, dim3(256), 0, st, part, mn, red, cstride, (float *)C);
  else
    hipLaunchKernelGGL((piece_reduce_kernel<uint16_t>), grid, dim3(256), 0, st, part, mn, red, cstride,
                       (uint16_t *)C);
  return launch_status("weight-gradient piece reduce");
}

// blocks of a tile kind resident on the chip at once: a 256 x 256 tile holds
// 128 KiB of LDS (one block per CU), the 128 x 128 tiles fit two per CU
static long resident_blocks(int tile) { return tile == TILE_256x256_W8 ? 256 : 512; }

// Split count of one dense weight-gradient product.  Splitting K only pays while
// the output tiles alone leave CUs idle: with `tiles` blocks of full depth
// already filling a round, s splits take ceil(s * tiles / resident) rounds of
// depth K / s (no shorter) plus a float32 reduction.  So take the largest s
// whose blocks still fit in one round (1 when the tiles alone fill it).
static int fill_split(long tiles, long resident, long max_by_depth) {  // 1 .. 8
  const long s = std::min<long>(resident / std::max<long>(tiles, 1), max_by_depth);
  return (int)std::max<long>(1, std::min<long>(s, 8));
}
// K windows for gemm_splitk: each at least 1024 deep
int splitk_count(bool f32, int M, int N, long K) {
  const int tile = f32 ? TILE_128x128 : (M >= 256 && N >= 256 ? TILE_256x256_W8 : TILE_128x128_W8);
  const long tiles = (long)((M + tile_rows(tile) - 1) / tile_rows(tile)) * col_tiles(EPI_PLAIN, tile, N);
  return fill_split(tiles, resident_blocks(tile), K / 1024);
}

size_t ffn_ws_bytes(const Shape &s) {
  const int esz = s.act_f32 ? 4 : 2;
  size_t b = align_up((size_t)s.R_max * s.dff * esz, 256);                       // hidden H
  if (s.n_shared) b += align_up((size_t)s.T * s.n_shared * s.dff * esz, 256);    // shared hidden
  b += align_up((size_t)4 * (s.E + 2) * 4, 256);                                  // tile prefixes
  return b;
}

template <typename TE>
static int ffn_typed(const Shape &s, const void *xin, const int32_t *gather, const int32_t *offsets,
                     const void *w1, const void *w3, const void *w2, void *y_perm, const void *x_shared,
                     const void *ws1, const void *ws3, const void *ws2, void *shared_out, void *ws, hipStream_t st,
                     const FoldOut &fold, void *gsave) {
  const int esz = sizeof(TE);
  char *p = (char *)ws;
  TE *H = (TE *)p;
  p += align_up((size_t)s.R_max * s.dff * esz, 256);
  TE *Hs = nullptr;
  const int fs = s.n_shared * s.dff;
  if (s.n_shared) {
    Hs = (TE *)p;
    p += align_up((size_t)s.T * fs * esz, 256);
  }
  int32_t *pre = (int32_t *)p;  // [launch][E+2]: tile prefixes of the (up to four) launches
  const bool glu = s.act == 1;
  const int has_x = s.n_shared ? 1 : 0;
  // narrow experts: the fused MLP (no hidden round trip through HBM)
  const bool fused = sizeof(TE) == 2 && mlp_fused_supported(s);
  if (fold.o && !(fused && fold_supported(s))) return -2;
  if (gsave && fused) return -2;  // the fused MLP keeps no pre-activations
  if (fused) {
    if (int rc = launch_mlp_fused(s, xin, gather, offsets, w1, w3, w2, y_perm, pre, st, fold)) return rc;
  }
  // f32 layers are parity-sized: the small tile is plenty
  const int tile = sizeof(TE) == 4 ? TILE_128x128 : pick_tile_routed(s);
  const int epi1 = glu ? EPI_SWIGLU : EPI_RELU;
  // the two GEMMs split their rows alike; only their tail tiles can differ
  Launch l[2], l2[2];
  const int nl = plan_launches(tile, epi1, s.dff, s.E, l);
  plan_launches(tile, EPI_PLAIN, s.dh, s.E, l2);

  GemmArgs a{};
  // ---- GEMM 1: H = act(x_perm W1^T [, x_perm W3^T])
  a.A = xin; a.lda = gather ? (long)s.H * s.dh : s.dh;
  a.gather = gather; a.gK = s.K; a.gEh = s.Eh; a.gdh = s.dh;
  a.B = w1; a.B2 = glu ? w3 : nullptr; a.ldb = s.dh; a.bstride = (long)s.dff * s.dh;
  a.C = H; a.ldc = s.dff;
  a.gsave = gsave; a.ldg = glu ? 2L * s.dff : s.dff;
  a.offsets = offsets; a.E = s.E; a.N = s.dff; a.K = s.dh; a.Mr_bound = s.R_max;
  a.has_x = 0; a.G = s.E;
  // ---- GEMM 2: y_perm = H W2^T
  GemmArgs b{};
  b.A = H; b.lda = s.dff;
  b.B = w2; b.B2 = nullptr; b.ldb = s.dff; b.bstride = (long)s.dh * s.dff;
  b.C = y_perm; b.ldc = s.dh;
  b.offsets = offsets; b.E = s.E; b.N = s.dh; b.K = s.dff; b.Mr_bound = s.R_max;
  b.has_x = 0; b.G = s.E;

  // one launch builds the tile prefixes of every routed launch of both GEMMs
  PrepArgs pa{};
  pa.offsets = offsets; pa.E = s.E; pa.has_x = 0; pa.Mx = 0; pa.prefix = pre;
  for (int i = 0; i < nl; ++i) {
    pa.c[i] = prep_cfg(epi1, l[i], a.N, 0);
    pa.c[nl + i] = prep_cfg(EPI_PLAIN, l2[i], b.N, 0);
  }
  for (int i = 0; i < nl && !fused; ++i) {
    if (i == 0) {
      hipLaunchKernelGGL(gemm_prep_kernel, dim3(2 * nl), dim3(1024), 0, st, pa);
      if (int rc = launch_status("gemm tile prefix")) return rc;
    }
    a.split = l[i].split;
    a.prefix = pre + (size_t)i * (s.E + 2);
    int rc = glu ? run_gemm_one<TE, EPI_SWIGLU>(a, l[i].tile, st) : run_gemm_one<TE, EPI_RELU>(a, l[i].tile, st);
    if (rc) return rc;
  }
  for (int i = 0; i < nl && !fused; ++i) {
    b.split = l2[i].split;
    b.prefix = pre + (size_t)(nl + i) * (s.E + 2);
    if (int rc = run_gemm_one<TE, EPI_PLAIN>(b, l2[i].tile, st)) return rc;
  }
  if (!has_x) return 0;

  // ---- shared experts ("MoE技术演进", "DeepSeekMoE" item 2): a plain
  // product over all T tokens, concatenated experts of width n_shared*d_ff,
  // in its own launches with tiles sized for T rows (in the routed launch
  // its tiles took the routed experts' small tile and ran at the end of the
  // tile list on two XCDs, re-reading its operands many times)
  const int tile_s = sizeof(TE) == 4 ? TILE_128x128 : pick_tile(s.T, 1);
  GemmArgs sa{};
  sa.E = 0; sa.has_x = 1; sa.G = 1;
  sa.Ax = x_shared; sa.ldax = s.d; sa.Bx = ws1; sa.Bx2 = glu ? ws3 : nullptr; sa.ldbx = s.d;
  sa.Cx = Hs; sa.ldcx = fs; sa.Mx = s.T; sa.Nx = fs; sa.Kx = s.d;
  int rc = glu ? run_plain<TE, EPI_SWIGLU>(sa, tile_s, st) : run_plain<TE, EPI_RELU>(sa, tile_s, st);
  if (rc) return rc;
  GemmArgs sb{};
  sb.E = 0; sb.has_x = 1; sb.G = 1;
  sb.Ax = Hs; sb.ldax = fs; sb.Bx = ws2; sb.Bx2 = nullptr; sb.ldbx = fs;
  sb.Cx = shared_out; sb.ldcx = s.d; sb.Mx = s.T; sb.Nx = s.d; sb.Kx = fs;
  return run_plain<TE, EPI_PLAIN>(sb, tile_s, st);
}

int launch_expert_ffn(const Shape &s, const void *xin, const int32_t *gather, const int32_t *offsets,
                      const void *w1, const void *w3, const void *w2, void *y_perm, const void *x_shared,
                      const void *ws1, const void *ws3, const void *ws2, void *shared_out, void *ws, hipStream_t st,
                      const FoldOut &fold, void *gsave) {
  if (s.act_f32)
    return ffn_typed<float>(s, xin, gather, offsets, w1, w3, w2, y_perm, x_shared, ws1, ws3, ws2, shared_out, ws, st,
                            fold, gsave);
  return ffn_typed<uint16_t>(s, xin, gather, offsets, w1, w3, w2, y_perm, x_shared, ws1, ws3, ws2, shared_out, ws,
                             st, fold, gsave);
}

bool ffn_grouped(const Shape &s) { return s.act_f32 || !mlp_fused_supported(s); }

size_t dense_ws_bytes() { return 0; }  // the tile counts come from the host

// C[M, N] = A[M, K] B[N, K]^T (+ residual): one plain group, its tile count
// known on the host (no prefix launch; a launch with no tiles is skipped)
int launch_dense(bool f32, const void *A, const void *B, void *C, const void *residual, int M, int N, int K,
                 void *ws, hipStream_t st) {
  (void)ws;
  GemmArgs a{};
  a.E = 0; a.has_x = 1; a.G = 1;
  a.Ax = A; a.ldax = K; a.Bx = B; a.ldbx = K; a.Cx = C; a.ldcx = N; a.Mx = M; a.Nx = N; a.Kx = K;
  a.res = residual; a.ldres = N;
  if (f32)
    return residual ? run_plain<float, EPI_RESID>(a, TILE_128x128, st) : run_plain<float, EPI_PLAIN>(a, TILE_128x128, st);
  const int tile = pick_tile(M, 1);
  return residual ? run_plain<uint16_t, EPI_RESID>(a, tile, st) : run_plain<uint16_t, EPI_PLAIN>(a, tile, st);
}

}  // namespace moe

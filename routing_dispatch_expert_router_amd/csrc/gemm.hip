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
// operands are K-contiguous.  Tiles: 128 x 128 outputs (SwiGLU: 128 rows x 64
// hidden columns, whose gate and up halves make the 128 B rows), k-chunk of
// 128 bytes, 4 waves each 64 x 64, LDS double buffer with XOR-swizzled 16-byte
// slots, one barrier per k-chunk.
#include "common.h"
#include "launch.h"

namespace moe {

enum { EPI_PLAIN = 0, EPI_RELU = 1, EPI_SWIGLU = 2, EPI_RESID = 3 };
constexpr int BM = 128, BN = 128;

struct GemmArgs {
  const void *A; long lda;                    // routed: A rows indexed by offsets
  const void *B; const void *B2; long ldb; long bstride;
  void *C; long ldc;
  const int32_t *offsets;
  int E, N, K;
  const void *Ax; long ldax;                  // extra group
  const void *Bx; const void *Bx2; long ldbx;
  void *Cx; long ldcx;
  int Mx, Nx, Kx, has_x;
  const void *res; long ldres;                // EPI_RESID: added to the extra group's output
  const int32_t *prefix;                      // [G+1] tile prefix
  int G;
};

template <int EPI> __host__ __device__ inline int n_tiles(int N) { return EPI == EPI_SWIGLU ? N / 64 : (N + BN - 1) / BN; }

// tile prefix over groups: tiles_g = ceil(M_g / BM) * n_tiles(N_g)
template <int EPI>
__global__ __launch_bounds__(1024) void gemm_prep_kernel(const int32_t *__restrict__ offsets, int E, int N,
                                                         int has_x, int Mx, int Nx, int32_t *__restrict__ prefix) {
  __shared__ int s[1024];
  const int G = E + has_x;
  const int tid = threadIdx.x;
  const int per = (G + 1023) / 1024;
  int loc[2] = {0, 0};
  int sum = 0;
  for (int i = 0; i < per && i < 2; ++i) {
    int g = tid * per + i;
    int v = 0;
    if (g < G) {
      int M = (g < E) ? offsets[g + 1] - offsets[g] : Mx;
      int nn = (g < E) ? N : Nx;
      v = (M + BM - 1) / BM * n_tiles<EPI>(nn);
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

template <typename TE, int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmArgs p) {
  constexpr int EPC = 16 / sizeof(TE);  // elements per 16-byte slot
  constexpr int BKE = 8 * EPC;          // elements per 128-byte k-chunk
  __shared__ u32x4 sA[2][BM * 8];
  __shared__ u32x4 sB[2][BN * 8];

  const int total = p.prefix[p.G];
  const int b = blockIdx.x;
  if (b >= total) return;
  // blocks go round-robin to the 8 XCDs; give each XCD a contiguous run of
  // tiles so tiles sharing operands share an L2
  const int q8 = total >> 3;
  const int lt = (b < 8 * q8) ? (b & 7) * q8 + (b >> 3) : b;
  int lo = 0, hi = p.G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (p.prefix[mid] <= lt) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  int local = lt - p.prefix[g];

  const TE *A, *B, *B2;
  TE *C;
  long lda, ldb, ldc;
  int M, N, K;
  if (g < p.E) {
    const int r0 = p.offsets[g];
    M = p.offsets[g + 1] - r0;
    lda = p.lda; ldb = p.ldb; ldc = p.ldc; N = p.N; K = p.K;
    A = (const TE *)p.A + (size_t)r0 * lda;
    B = (const TE *)p.B + (size_t)g * p.bstride;
    B2 = p.B2 ? (const TE *)p.B2 + (size_t)g * p.bstride : nullptr;
    C = (TE *)p.C + (size_t)r0 * ldc;
  } else {
    M = p.Mx; N = p.Nx; K = p.Kx;
    lda = p.ldax; ldb = p.ldbx; ldc = p.ldcx;
    A = (const TE *)p.Ax; B = (const TE *)p.Bx; B2 = (const TE *)p.Bx2; C = (TE *)p.Cx;
  }
  // grouped raster inside the group: bands of GM m-tiles, n outer, m inner
  const int mt = (M + BM - 1) / BM, nt = n_tiles<EPI>(N);
  constexpr int GM = 8;
  const int band = local / (GM * nt);
  const int first_m = band * GM;
  const int gsm = min(mt - first_m, GM);
  const int in_band = local - band * GM * nt;
  const int tm = first_m + in_band % gsm;
  const int tn = in_band / gsm;
  const int m0 = tm * BM;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wm = wv >> 1, wn = wv & 1;
  const int cq = lane >> 4, l16 = lane & 15;

  // global -> LDS assignment: 1024 16-byte slots per operand tile, 4 per thread
  const TE *pa[4];
  const TE *pb[4];
  int slot[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 3) + 32 * i, q = tid & 7;
    slot[i] = row * 8 + (q ^ (row & 7));
    pa[i] = A + (size_t)min(m0 + row, M - 1) * lda + q * EPC;
    if (EPI == EPI_SWIGLU) {
      const int hn = tn * 64 + (row & 63);
      pb[i] = ((row < 64) ? B : B2) + (size_t)hn * ldb + q * EPC;
    } else {
      pb[i] = B + (size_t)min(tn * BN + row, N - 1) * ldb + q * EPC;
    }
  }
  const int nk = K / BKE;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[4], rb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = *reinterpret_cast<const u32x4 *>(pa[i]);
    rb[i] = *reinterpret_cast<const u32x4 *>(pb[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sA[0][slot[i]] = ra[i];
    sB[0][slot[i]] = rb[i];
  }
  __syncthreads();

  // B-tile row of this wave's n-fragment f
  int brow[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
    brow[f] = (EPI == EPI_SWIGLU) ? ((f < 2) ? wn * 32 + f * 16 : 64 + wn * 32 + (f - 2) * 16) + l16
                                  : wn * 64 + f * 16 + l16;

  for (int kc = 0; kc < nk; ++kc) {
    const int st = kc & 1;
    if (kc + 1 < nk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const u32x4 *>(pa[i] + (size_t)(kc + 1) * BKE);
        rb[i] = *reinterpret_cast<const u32x4 *>(pb[i] + (size_t)(kc + 1) * BKE);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int qs = cq + 4 * ks;
      u32x4 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + l16;
        fa[i] = sA[st][r * 8 + (qs ^ (r & 7))];
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) fb[f] = sB[st][brow[f] * 8 + (qs ^ (brow[f] & 7))];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[i][f] = mma16(fa[i], fb[f], acc[i][f], TE());
    }
    if (kc + 1 < nk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sA[st ^ 1][slot[i]] = ra[i];
        sB[st ^ 1][slot[i]] = rb[i];
      }
    }
    __syncthreads();
  }

  // epilogue: acc[i][f][v] = C[wm*64 + i*16 + 4*cq + v][n-fragment f, column l16]
  const TE *R = (EPI == EPI_RESID) ? (const TE *)p.res : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + wm * 64 + i * 16 + 4 * cq + v;
      if (row >= M) continue;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int col = tn * 64 + wn * 32 + f * 16 + l16;
          const float gt = acc[i][f][v], up = acc[i][f + 2][v];
          const float h = gt / (1.0f + __expf(-gt)) * up;
          C[(size_t)row * ldc + col] = Elem<TE>::from_f32(h);
        }
      } else {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = tn * BN + wn * 64 + f * 16 + l16;
          if (col >= N) continue;
          float o = acc[i][f][v];
          if (EPI == EPI_RELU) o = fmaxf(o, 0.0f);
          if (EPI == EPI_RESID) o += Elem<TE>::to_f32(R[(size_t)row * p.ldres + col]);
          C[(size_t)row * ldc + col] = Elem<TE>::from_f32(o);
        }
      }
    }
}

// ---------------------------------------------------------------- host
static long max_tiles(long rows_bound, int groups, int n_tiles_) {
  return ((rows_bound + BM - 1) / BM + groups) * n_tiles_;
}

template <typename TE, int EPI>
static int run_gemm(GemmArgs a, long grid, int prepN, int prepNx, int32_t *prefix, hipStream_t st) {
  a.prefix = prefix;
  hipLaunchKernelGGL((gemm_prep_kernel<EPI>), dim3(1), dim3(1024), 0, st, a.offsets, a.E, prepN, a.has_x, a.Mx,
                     prepNx, prefix);
  if (hipGetLastError() != hipSuccess) return -4;
  if (grid <= 0) return 0;
  hipLaunchKernelGGL((grouped_gemm_kernel<TE, EPI>), dim3(grid), dim3(256), 0, st, a);
  if (hipGetLastError() != hipSuccess) return -4;
  return 0;
}

size_t ffn_ws_bytes(const Shape &s) {
  const int esz = s.act_f32 ? 4 : 2;
  size_t b = align_up((size_t)s.R_max * s.dff * esz, 256);                       // hidden H
  if (s.n_shared) b += align_up((size_t)s.T * s.n_shared * s.dff * esz, 256);    // shared hidden
  b += 2 * align_up((size_t)(s.E + 2) * 4, 256);                                  // tile prefixes
  return b;
}

template <typename TE>
static int ffn_typed(const Shape &s, const void *x_perm, const int32_t *offsets, const void *w1, const void *w3,
                     const void *w2, void *y_perm, const void *x_shared, const void *ws1, const void *ws3,
                     const void *ws2, void *shared_out, void *ws, hipStream_t st) {
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
  int32_t *pre1 = (int32_t *)p;
  p += align_up((size_t)(s.E + 2) * 4, 256);
  int32_t *pre2 = (int32_t *)p;
  const bool glu = s.act == 1;
  const int has_x = s.n_shared ? 1 : 0;

  GemmArgs a{};
  // ---- GEMM 1: H = act(x_perm W1^T [, x_perm W3^T])
  a.A = x_perm; a.lda = s.dh;
  a.B = w1; a.B2 = glu ? w3 : nullptr; a.ldb = s.dh; a.bstride = (long)s.dff * s.dh;
  a.C = H; a.ldc = s.dff;
  a.offsets = offsets; a.E = s.E; a.N = s.dff; a.K = s.dh;
  a.has_x = has_x;
  if (has_x) {
    a.Ax = x_shared; a.ldax = s.d; a.Bx = ws1; a.Bx2 = glu ? ws3 : nullptr; a.ldbx = s.d;
    a.Cx = Hs; a.ldcx = fs; a.Mx = s.T; a.Nx = fs; a.Kx = s.d;
  }
  a.G = s.E + has_x;
  int rc;
  if (glu) {
    long grid = max_tiles(s.R_max, s.E, n_tiles<EPI_SWIGLU>(s.dff)) +
                (has_x ? max_tiles(s.T, 0, n_tiles<EPI_SWIGLU>(fs)) : 0);
    rc = run_gemm<TE, EPI_SWIGLU>(a, grid, s.dff, fs, pre1, st);
  } else {
    long grid = max_tiles(s.R_max, s.E, n_tiles<EPI_RELU>(s.dff)) +
                (has_x ? max_tiles(s.T, 0, n_tiles<EPI_RELU>(fs)) : 0);
    rc = run_gemm<TE, EPI_RELU>(a, grid, s.dff, fs, pre1, st);
  }
  if (rc) return rc;
  // ---- GEMM 2: y_perm = H W2^T ; shared_out = Hs Ws2^T
  GemmArgs b{};
  b.A = H; b.lda = s.dff;
  b.B = w2; b.B2 = nullptr; b.ldb = s.dff; b.bstride = (long)s.dh * s.dff;
  b.C = y_perm; b.ldc = s.dh;
  b.offsets = offsets; b.E = s.E; b.N = s.dh; b.K = s.dff;
  b.has_x = has_x;
  if (has_x) {
    b.Ax = Hs; b.ldax = fs; b.Bx = ws2; b.Bx2 = nullptr; b.ldbx = fs;
    b.Cx = shared_out; b.ldcx = s.d; b.Mx = s.T; b.Nx = s.d; b.Kx = fs;
  }
  b.G = s.E + has_x;
  long grid2 = max_tiles(s.R_max, s.E, n_tiles<EPI_PLAIN>(s.dh)) +
               (has_x ? max_tiles(s.T, 0, n_tiles<EPI_PLAIN>(s.d)) : 0);
  return run_gemm<TE, EPI_PLAIN>(b, grid2, s.dh, s.d, pre2, st);
}

int launch_expert_ffn(const Shape &s, const void *x_perm, const int32_t *offsets, const void *w1, const void *w3,
                      const void *w2, void *y_perm, const void *x_shared, const void *ws1, const void *ws3,
                      const void *ws2, void *shared_out, void *ws, hipStream_t st) {
  if (s.act_f32)
    return ffn_typed<float>(s, x_perm, offsets, w1, w3, w2, y_perm, x_shared, ws1, ws3, ws2, shared_out, ws, st);
  return ffn_typed<uint16_t>(s, x_perm, offsets, w1, w3, w2, y_perm, x_shared, ws1, ws3, ws2, shared_out, ws, st);
}

size_t dense_ws_bytes() { return 256; }

int launch_dense(bool f32, const void *A, const void *B, void *C, const void *residual, int M, int N, int K,
                 void *ws, hipStream_t st) {
  GemmArgs a{};
  a.E = 0; a.has_x = 1; a.G = 1;
  a.Ax = A; a.ldax = K; a.Bx = B; a.ldbx = K; a.Cx = C; a.ldcx = N; a.Mx = M; a.Nx = N; a.Kx = K;
  a.res = residual; a.ldres = N;
  long grid = max_tiles(M, 0, n_tiles<EPI_PLAIN>(N));
  int32_t *pre = (int32_t *)ws;
  if (f32)
    return residual ? run_gemm<float, EPI_RESID>(a, grid, 0, N, pre, st) : run_gemm<float, EPI_PLAIN>(a, grid, 0, N, pre, st);
  return residual ? run_gemm<uint16_t, EPI_RESID>(a, grid, 0, N, pre, st)
                  : run_gemm<uint16_t, EPI_PLAIN>(a, grid, 0, N, pre, st);
}

}  // namespace moe

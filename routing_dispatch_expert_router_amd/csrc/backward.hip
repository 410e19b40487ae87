// Layer backward: the elementwise, permutation and router kernels (the
// products run on the grouped GEMM, gemm.hip).
//
// Gradients of <dy, y> + lam * l_aux with the forward's decisions held fixed,
// by the chain rule through the definitions the forward follows: y_t = x_t +
// s_t + sum_kept g_{t,j} F_e(x_t) ("MoE技术演进", "DeepSeekMoE" items 1-2,
// "GShard" item 3); F_e = W2 (SiLU(W1 v) * W3 v) ("大语言模型并行策略（七）：专家
// 并行", "MoE 模型的参数量分析"); g = softmax(W_r x + b) at the chosen experts,
// optionally renormalised ("MoE技术演进", "Adaptive Mixtures of Local Experts"
// gating equation, "DeepSeekMoE" item 1); l_aux = sum_e m_e c_e / S ("GShard"
// item 1).  Every reduction runs in a fixed order (bit-reproducible).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

__global__ void zero_f32_kernel(float *p, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) p[i] = 0.f;
}

// ---------------------------------------------------------------- per kept row
// dg[a] = <dy_{t,h}, y_perm_r> and dY_r = g_a * dy_{t,h} for row r holding
// assignment a = t*K + j on expert e of head h = e / E_h (dy_{t,h}: columns
// [h*dh, (h+1)*dh) of row t).  W lanes per row (W = the row's 16-byte chunks,
// at most 64), 64 / W rows per wave; dg of dropped assignments stays 0.
template <typename TA, int W>
__global__ __launch_bounds__(256) void bwd_rows_kernel(const TA *__restrict__ dy, const TA *__restrict__ y_perm,
                                                       const float *__restrict__ gates,
                                                       const int32_t *__restrict__ src_of,
                                                       const int32_t *__restrict__ topk_idx,
                                                       const int32_t *__restrict__ offsets, int E, int Eh, int K,
                                                       int dh, long ld_dy, TA *__restrict__ dY,
                                                       float *__restrict__ dg) {
  constexpr int EPC = 16 / sizeof(TA);
  const int r = (blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / W) + (threadIdx.x & 63) / W;
  const int lane = threadIdx.x & (W - 1);
  if (r >= offsets[E]) return;  // whole groups of W lanes: the sum below stays inside a group
  const int a = src_of[r], t = a / K, h = topk_idx[a] / Eh;
  const float g = gates[a];
  const u32x4 *s = (const u32x4 *)(dy + (size_t)t * ld_dy + (size_t)h * dh);
  const u32x4 *yp = (const u32x4 *)(y_perm + (size_t)r * dh);
  u32x4 *o = (u32x4 *)(dY + (size_t)r * dh);
  float dot = 0.f;
  for (int c = lane; c < dh / EPC; c += W) {
    const u32x4 vs = s[c], vy = yp[c];
    u32x4 vo;
    if constexpr (sizeof(TA) == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float s0 = bf16_to_f32((uint16_t)(vs[q] & 0xFFFFu)), s1 = bf16_to_f32((uint16_t)(vs[q] >> 16));
        const float y0 = bf16_to_f32((uint16_t)(vy[q] & 0xFFFFu)), y1 = bf16_to_f32((uint16_t)(vy[q] >> 16));
        dot += s0 * y0;
        dot += s1 * y1;
        vo[q] = (uint32_t)f32_to_bf16(g * s0) | ((uint32_t)f32_to_bf16(g * s1) << 16);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float s0 = __uint_as_float(vs[q]);
        dot += s0 * __uint_as_float(vy[q]);
        vo[q] = __float_as_uint(g * s0);
      }
    }
    o[c] = vo;
  }
  dot = group_sum_fixed(dot, W);
  if (lane == 0) dg[a] = dot;
}

// ---------------------------------------------------------------- expert padding
// poff[e] = sum_{e' < e} roundup(counts[e'], 64): expert e's rows occupy
// columns [poff[e], poff[e] + counts[e]) of the transposed activations, the
// rest of its 64-aligned range is zero.  One block.
__global__ __launch_bounds__(1024) void bwd_poff_kernel(const int32_t *__restrict__ offsets, int E,
                                                        int32_t *__restrict__ poff) {
  __shared__ int s[1024];
  const int tid = threadIdx.x, per = (E + 1023) / 1024;
  int sum = 0, loc[8];
  for (int i = 0; i < per && i < 8; ++i) {
    const int e = tid * per + i;
    const int v = e < E ? (offsets[e + 1] - offsets[e] + 63) / 64 * 64 : 0;
    loc[i] = v;
    sum += v;
  }
  s[tid] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int u = tid >= o ? s[tid - o] : 0;
    __syncthreads();
    s[tid] += u;
    __syncthreads();
  }
  int run = s[tid] - sum;
  for (int i = 0; i < per && i < 8; ++i) {
    const int e = tid * per + i;
    if (e < E) poff[e] = run;
    run += loc[i];
  }
  if (tid == 1023) poff[E] = s[1023];
}

// pmap_r[j] = row r held by padded column j (or -1); pmap_x[j] = t*H + h for
// its token t and head h: the row of the expert input viewed as [T*H, dh]
__global__ void bwd_pmap_kernel(const int32_t *__restrict__ offsets, const int32_t *__restrict__ poff,
                                const int32_t *__restrict__ src_of, int E, int Eh, int H, int K, long npad,
                                int32_t *__restrict__ pmap_r, int32_t *__restrict__ pmap_x) {
  for (long j = blockIdx.x * (long)blockDim.x + threadIdx.x; j < npad; j += (long)gridDim.x * blockDim.x) {
    int r = -1, e = 0;
    if (j < poff[E]) {
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (poff[mid] <= j) lo = mid; else hi = mid - 1;
      }
      const int rr = offsets[lo] + (int)(j - poff[lo]);
      if (rr < offsets[lo + 1]) r = rr;
      e = lo;
    }
    pmap_r[j] = r;
    pmap_x[j] = r >= 0 ? (src_of[r] / K) * H + e / Eh : -1;
  }
}

// ---------------------------------------------------------------- transpose
// dst[b][c][j] = source row j's column (coff + c), for c < ncols, j < njcols:
//   rmap: source row rmap[j] (zero when -1); else row j when j < nvalid (zero after).
// kchunk: dst k-chunked for the K-grouped products, (c, j) at (j / KC) * ld_dst *
// KC + c * KC + j % KC with KC the elements of 128 bytes (ld_dst = rows of dst),
// so one k-step of a product tile reads a contiguous block; else row-major.
// Tiles of 64 columns x 64 rows through LDS, 16-byte global accesses both ways.
template <typename TA>
__global__ __launch_bounds__(256) void transpose_kernel(const TA *__restrict__ src, long ld_src, long bs_src,
                                                        const int32_t *__restrict__ rmap, long nvalid, long njcols,
                                                        int ncols, int coff, TA *__restrict__ dst, long ld_dst,
                                                        long bs_dst, int kchunk) {
  constexpr int KC = 128 / sizeof(TA);
  constexpr int EPC = 16 / sizeof(TA), CH = 64 / EPC;  // 16-byte chunks per 64 elements
  __shared__ TA tile[64][64 + EPC];
  const long j0 = (long)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  src += (size_t)blockIdx.z * bs_src;
  dst += (size_t)blockIdx.z * bs_dst;
  for (int i = threadIdx.x; i < 64 * CH; i += 256) {
    const int jj = i / CH, ch = i % CH;
    const long j = j0 + jj;
    long row = -1;
    if (j < njcols) row = rmap ? (long)rmap[j] : (j < nvalid ? j : -1);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row >= 0 && c0 + ch * EPC < ncols) v = *(const u32x4 *)(src + (size_t)row * ld_src + coff + c0 + ch * EPC);
    const TA *pv = (const TA *)&v;
#pragma unroll
    for (int q = 0; q < EPC; ++q) tile[jj][ch * EPC + q] = pv[q];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * CH; i += 256) {
    const int cc = i / CH, ch = i % CH;
    if (c0 + cc >= ncols || j0 + ch * EPC >= njcols) continue;
    u32x4 v;
    TA *pv = (TA *)&v;
#pragma unroll
    for (int q = 0; q < EPC; ++q) pv[q] = tile[ch * EPC + q][cc];
    const long j = j0 + ch * EPC;
    const size_t o = kchunk ? (size_t)(j / KC) * ld_dst * KC + (size_t)(c0 + cc) * KC + j % KC
                            : (size_t)(c0 + cc) * ld_dst + j;
    *(u32x4 *)(dst + o) = v;
  }
}

// ---------------------------------------------------------------- router
// dl[t][e] = p_e (dp_e - sum_e' p_e' dp_e') over the head's E_h experts,
// p = the head's softmax of the logits; dp from the gate gradients of the
// head's k slots (renormalised: (dg_j - sum dg g) / P at the chosen experts)
// plus lam * demand_e / T^2 (aux loss, one head) plus seq_w * c_{s,e} / L^2 for
// the token's sequence s (sequence-wise balance term, one head).  W lanes per
// (token, head) (W a power of two, at least min(E_h, 64)), 64 / W pairs per wave.
template <int W>
__global__ __launch_bounds__(256) void router_bwd_kernel(const float *__restrict__ logits,
                                                         const int32_t *__restrict__ topk_idx,
                                                         const float *__restrict__ gates,
                                                         const float *__restrict__ dg,
                                                         const int32_t *__restrict__ demand, int T, int H, int E,
                                                         int Eh, int K, int k, int renorm, float lam,
                                                         const int32_t *__restrict__ seq_cnt, int L, float seq_w,
                                                         float *__restrict__ dl) {
  const long pair = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / W) + ((threadIdx.x & 63) / W);
  const int lane = threadIdx.x & (W - 1);
  if (pair >= (long)T * H) return;  // whole groups of W lanes: the shuffles below stay inside a group
  const int t = (int)(pair / H), h = (int)(pair % H);
  const float *l = logits + (size_t)t * E + (size_t)h * Eh;
  const int32_t *ti = topk_idx + (size_t)t * K + (size_t)h * k;
  const float *tg = gates + (size_t)t * K + (size_t)h * k;
  const float *tdg = dg + (size_t)t * K + (size_t)h * k;
  float m = -INFINITY;
  for (int e = lane; e < Eh; e += W) m = fmaxf(m, l[e]);
  m = wave_max(m, W);
  float z = 0.f;
  for (int e = lane; e < Eh; e += W) z += __expf(l[e] - m);
  z = group_sum_fixed(z, W);
  // chosen experts: P = sum p, S = sum dg * g
  float P = 0.f, sdg = 0.f;
  for (int j = 0; j < k; ++j) {
    const int e = ti[j] - h * Eh;
    P += __expf(l[e] - m) / z;
    sdg += tdg[j] * tg[j];
  }
  const float invT2 = 1.0f / ((float)T * (float)T);
  const float invL2 = seq_cnt ? 1.0f / ((float)L * (float)L) : 0.f;
  const int32_t *sc = seq_cnt ? seq_cnt + (size_t)(t / L) * E : nullptr;
  auto dp_of = [&](int e) {
    float dp = lam * (float)demand[h * Eh + e] * invT2;
    if (sc) dp += seq_w * (float)sc[h * Eh + e] * invL2;
    for (int j = 0; j < k; ++j)
      if (ti[j] - h * Eh == e) dp += renorm ? (tdg[j] - sdg) / P : tdg[j];
    return dp;
  };
  // dp_e for this lane's experts, then sum p * dp
  float spdp = 0.f;
  for (int e = lane; e < Eh; e += W) spdp += __expf(l[e] - m) / z * dp_of(e);
  spdp = group_sum_fixed(spdp, W);
  for (int e = lane; e < Eh; e += W) dl[(size_t)t * E + (size_t)h * Eh + e] = __expf(l[e] - m) / z * (dp_of(e) - spdp);
}

// ---------------------------------------------------------------- float32 tile
// acc += sum_{k in [k_beg, k_end)} a(k, m) b(k, n) for the 64 x 64 output tile at
// (m0, n0); thread (tm, tn) = (tid / 16, tid % 16) owns m0 + 4 tm + i, n0 + 4 tn + j.
// b(k, n) = B[k ldb + n]; a(k, m) = A[k lda + m], or A[m lda + k] when A_MK (the
// operand is staged transposed into LDS).  k ascends: the order is fixed.
struct TileSmem {
  __align__(16) float a[32][68];
  __align__(16) float b[32][68];
};

template <bool A_MK, typename TA_, typename TB_>
__device__ __forceinline__ void tile_outer(float (&acc)[4][4], TileSmem &sm, const TA_ *__restrict__ A, long lda,
                                           int M, const TB_ *__restrict__ B, long ldb, int N, int m0, int n0,
                                           int k_beg, int k_end) {
  const int tid = threadIdx.x, tm = tid >> 4, tn = tid & 15;
  for (int k0 = k_beg; k0 < k_end; k0 += 32) {
    const int nk = min(32, k_end - k0);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i = tid + 256 * r;
      int kk, mm;
      if (A_MK) {
        kk = i & 31;
        mm = i >> 5;
      } else {
        kk = i >> 6;
        mm = i & 63;
      }
      float av = 0.f;
      if (kk < nk && m0 + mm < M)
        av = Elem<TA_>::to_f32(A_MK ? A[(size_t)(m0 + mm) * lda + k0 + kk] : A[(size_t)(k0 + kk) * lda + m0 + mm]);
      sm.a[kk][mm] = av;
      const int kb = i >> 6, nb = i & 63;
      sm.b[kb][nb] = (kb < nk && n0 + nb < N) ? Elem<TB_>::to_f32(B[(size_t)(k0 + kb) * ldb + n0 + nb]) : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < nk; ++kk) {
      const float4 av = *(const float4 *)&sm.a[kk][4 * tm];
      const float4 bv = *(const float4 *)&sm.b[kk][4 * tn];
      const float am[4] = {av.x, av.y, av.z, av.w}, bn[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += am[i] * bn[j];
    }
    __syncthreads();
  }
}

// dW_r = dl^T u in float32, per head h: rows [h*E_h, (h+1)*E_h) of dW_r from
// the head's dl columns and u's h-th slice (m = expert, n = column, k = token).
// Block (eb, cb, h*nsplit + ts) covers token range ts and writes
// part[ts][e][c]; a second pass adds the ranges in ascending order (fixed
// order: reproducible).
template <typename TX>
__global__ __launch_bounds__(256) void router_wgrad_kernel(const float *__restrict__ dl, const TX *__restrict__ x,
                                                           long ldx, int T, int E, int Eh, int dh, int nsplit,
                                                           float *__restrict__ part) {
  __shared__ TileSmem sm;
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const int h = blockIdx.z / nsplit, ts = blockIdx.z % nsplit;
  const int per = (T + nsplit - 1) / nsplit;
  const int t_beg = min(T, ts * per), t_end = min(T, t_beg + per);
  float acc[4][4] = {};
  tile_outer<false>(acc, sm, dl + (size_t)h * Eh, E, Eh, x + (size_t)h * dh, ldx, dh, m0, n0, t_beg, t_end);
  const int tm = threadIdx.x >> 4, tn = threadIdx.x & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = m0 + 4 * tm + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = n0 + 4 * tn + j;
      if (e < Eh && c < dh) part[((size_t)ts * E + (size_t)h * Eh + e) * dh + c] = acc[i][j];
    }
  }
}

// dw = sum of the nsplit partials in ascending order; n is a multiple of 4
// (d_head is a multiple of 64).  Four columns per thread, eight partials'
// loads in flight at a time (the adds keep the ascending order).
__global__ void router_wgrad_sum_kernel(const float *__restrict__ part, long n, int nsplit, float *__restrict__ dw) {
  const long n4 = n / 4;
  const float4 *p4 = (const float4 *)part;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n4; i += (long)gridDim.x * blockDim.x) {
    float4 s = p4[i];
    int ts = 1;
    for (; ts + 8 <= nsplit; ts += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p4[(size_t)(ts + u) * n4 + i];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
      }
    }
    for (; ts < nsplit; ++ts) {
      const float4 v = p4[(size_t)ts * n4 + i];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    ((float4 *)dw)[i] = s;
  }
}

// ---------------------------------------------------------------- router weight gradient on MFMA (bf16 layers)
// The contraction runs over tokens, which neither operand holds contiguously:
// dl is [T][E] and x is [T][H*dh].  dl is small, so a first pass rewrites it
// token-contiguous as three bf16 planes (hi = bf16(v), mid = bf16(v - hi),
// lo = bf16(v - hi - mid); each difference is exact in float32, so the three
// sum to v within about 2^-24 |v|).  bf16 x bf16 products are exact in float32,
// so the MFMA product with float32 accumulation keeps the float32 result.  x
// stays where it is: its rows go to LDS as they are and transposing LDS reads
// (ds_read_b64_tr_b16) hand each lane the k values it needs.
//
// A transposing read gives lane group q (lanes 16q .. 16q+15) the tokens
// 4q .. 4q+3 and 16+4q .. 16+4q+3 of a 32-token step.  A plain 16-byte read of
// a token-contiguous row gives lane group q positions 8q .. 8q+7, so the
// planes store, within every 32-token block, position 8q + j = token 4q + j
// (j < 4) or 16 + 4q + j - 4 (j >= 4): both operands then agree on the token
// of every byte a lane feeds to the MFMA.
__device__ __forceinline__ int rw_token_of_pos(int pos) {  // 0 <= pos < 32
  const int q = pos >> 3, j = pos & 7;
  return j < 4 ? 4 * q + j : 12 + 4 * q + j;
}

// planes[h][p][e][t'] (e < ep, t' < tp; zero past T and past E_h).  Block
// (64-token chunk, 64 experts, head): dl staged through LDS (coalesced reads),
// each thread then writes 8 positions (16 bytes) of one expert per plane.
__global__ __launch_bounds__(256) void router_dl_planes_kernel(const float *__restrict__ dl, int T, int E, int Eh,
                                                               int ep, int tp, uint16_t *__restrict__ planes) {
  __shared__ float sv[64][65];
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64, h = blockIdx.z;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63, t = t0 + r, e = e0 + c;
    sv[r][c] = (t < T && e < Eh) ? dl[(size_t)t * E + (size_t)h * Eh + e] : 0.f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int c = i >> 3, g = i & 7, e = e0 + c;  // expert, group of 8 positions in the chunk
    if (e >= ep) continue;
    uint32_t w[3][4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      uint32_t pk[3] = {0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int pos = 8 * (g & 3) + j + u;
        const float v = sv[32 * (g >> 2) + rw_token_of_pos(pos)][c];
        const uint16_t b0 = f32_to_bf16(v);
        const float r1 = v - bf16_to_f32(b0);
        const uint16_t b1 = f32_to_bf16(r1);
        const uint16_t b2 = f32_to_bf16(r1 - bf16_to_f32(b1));
        pk[0] |= (uint32_t)b0 << (16 * u);
        pk[1] |= (uint32_t)b1 << (16 * u);
        pk[2] |= (uint32_t)b2 << (16 * u);
      }
#pragma unroll
      for (int p = 0; p < 3; ++p) w[p][j >> 1] = pk[p];
    }
#pragma unroll
    for (int p = 0; p < 3; ++p)
      *(u32x4 *)(planes + (((size_t)h * 3 + p) * ep + e) * tp + t0 + 8 * g) = u32x4{w[p][0], w[p][1], w[p][2], w[p][3]};
  }
}

// x rows in LDS: 64 token rows of 256 columns (512 bytes) per stage, stored as
// 32 row pairs of 1056 bytes (two rows + 32 bytes of padding), so pair j starts
// at bank 8 * (j % 8): the 16 rows one transposing read covers spread over all
// banks, two rows per bank, the minimum for 512 bytes.  One direct-load
// instruction (64 lanes x 16 bytes) fills one pair.
constexpr int RW_PAIR = 1056, RW_BSTAGE = 32 * RW_PAIR;
__device__ __forceinline__ int rw_rowoff(int r) { return (r >> 1) * RW_PAIR + (r & 1) * 512; }
typedef short rw_v4s __attribute__((ext_vector_type(4)));

// part[ts][h*E_h + e][c] = sum over tokens t of range ts of dl[t][h*E_h + e] *
// x[t][h*dh + c].  Block tile: BM experts (all three planes) x 256 columns; 4
// waves side by side in n (64 columns each, BM/16 x 4 fragments of 16 x 16);
// 64-token chunks in a two-stage ring.  The planes' rows (128 bytes per chunk)
// use the 16-byte-slot XOR swizzle of the grouped GEMM and plain ds_read_b128.
// Tiles go to XCDs in contiguous runs, experts fastest, so the tiles that read
// the same x columns share an L2.
template <int BM>
__global__ __launch_bounds__(256) void router_wgrad_mfma_kernel(const uint16_t *__restrict__ planes,
                                                                const uint16_t *__restrict__ x, long ldx, int T,
                                                                int tp, int E, int Eh, int ep, int dh, int H, int per,
                                                                int nsplit, float *__restrict__ part) {
  constexpr int MF = BM / 16, SA = 3 * BM * 8;  // A: 16-byte slots per stage (3 planes x BM rows x 8)
  constexpr int LA = (SA + 255) / 256, LAMIN = SA / 256, LB = 8;
  static_assert(SA % 64 == 0, "whole waves of A slots");
  extern __shared__ u32x4 rw_smem[];
  u32x4 *sA = rw_smem;                                // [2][SA]
  char *sB = (char *)(rw_smem + 2 * SA);              // [2][RW_BSTAGE]

  const int mt = ep / BM, nt = (dh + 255) / 256;
  const int total = mt * nt * nsplit * H;
  const int b = blockIdx.x;
  const int q8 = total >> 3;
  const int lt = (b < 8 * q8) ? (b & 7) * q8 + (b >> 3) : b;
  const int tm = lt % mt, tn = (lt / mt) % nt, ts = (lt / (mt * nt)) % nsplit, h = lt / (mt * nt * nsplit);
  const int m0 = tm * BM, n0 = tn * 256;
  const int t_beg = min(T, ts * per), t_end = min(T, t_beg + per), klen = t_end - t_beg;
  const int nk = (klen + 63) / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int gq = lane >> 4, li = lane & 15;

  // A: slot s = i*256 + tid holds chunk swz(row, s % 8) of plane row `row`
  const uint16_t *asrc[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int s = min(i * 256 + tid, SA - 1), row = s >> 3, q = (s & 7) ^ (row & 7);
    const int p = row / BM, e = m0 + row % BM;
    asrc[i] = planes + (((size_t)h * 3 + p) * ep + e) * tp + t_beg + 8 * q;
  }
  // B: instruction i of wave wv fills pair j = 4i + wv; lane -> row 2j + lane/32,
  // columns 8*(lane % 32) .. +7 (clamped into the head: duplicates, never stored)
  const int lrow = lane >> 5, lcol = min(n0 + (lane & 31) * 8, dh - 8);
  const uint16_t *xb = x + (size_t)h * dh + lcol;
  auto issue = [&](int kc, int st) {
#pragma unroll
    for (int i = 0; i < LA; ++i)
      if (i * 256 + wv * 64 < SA) load_lds16(asrc[i] + kc * 64, sA + st * SA + i * 256 + wv * 64);
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int j = 4 * i + wv;
      const int t = min(t_beg + kc * 64 + 2 * j + lrow, T - 1);  // rows past T: re-read, zeroed below
      load_lds16(xb + (size_t)t * ldx, sB + st * RW_BSTAGE + j * RW_PAIR);
    }
  };

  f32x4 acc[MF][4];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  // per lane: byte offsets of its two transposing reads of k-step ks (column 0 of the wave)
  int roff[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      roff[ks][hh] = rw_rowoff(32 * ks + 16 * hh + 4 * gq + (li >> 2)) + 8 * (li & 3) + 2 * 64 * wv;
  auto fragb = [&](const char *stage, int ks, int f) -> u32x4 {
    const rw_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) rw_v4s *)(stage + roff[ks][0] + 32 * f));
    const rw_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) rw_v4s *)(stage + roff[ks][1] + 32 * f));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
  };
  // zero the tokens at or past the range's end (last chunk only): element w
  // of a fragment holds tokens kb + 2w, kb + 2w + 1 (w < 2) or kb + 12 + 2w, +1
  auto maskb = [&](u32x4 &fr, int kc, int ks) {
    const int kb = kc * 64 + 32 * ks + 4 * gq;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int k = kb + (w < 2 ? 2 * w : 12 + 2 * w);
      fr[w] &= ((k < klen) ? 0xFFFFu : 0u) | ((k + 1 < klen) ? 0xFFFF0000u : 0u);
    }
  };
  auto readk = [&](int kc, int ks, u32x4 (&fa)[3][MF], u32x4 (&fb)[4]) {
    const u32x4 *st = sA + (kc & 1) * SA;
    const int sw = (gq + 4 * ks) ^ (li & 7);
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int i = 0; i < MF; ++i) fa[p][i] = st[(p * BM + i * 16 + li) * 8 + sw];
    const bool last = kc == nk - 1 && (klen & 63);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      fb[f] = fragb(sB + (kc & 1) * RW_BSTAGE, ks, f);
      if (last) maskb(fb[f], kc, ks);
    }
  };
  auto mfma = [&](const u32x4 (&fa)[3][MF], const u32x4 (&fb)[4]) {
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[i][f] = mma16(fb[f], fa[p][i], acc[i][f], uint16_t());
  };

  if (nk > 0) {
    issue(0, 0);
    if (nk > 1) {
      issue(1, 1);
      wait_vmcnt<LAMIN + LB>();  // chunk 0 landed (a wave with more A slots also waits for one of chunk 1)
    } else {
      wait_vmcnt0();
    }
    __syncthreads();
    u32x4 fa0[3][MF], fb0[4], fa1[3][MF], fb1[4];
    readk(0, 0, fa0, fb0);
    for (int kc = 0; kc < nk; ++kc) {
      readk(kc, 1, fa1, fb1);
      mfma(fa0, fb0);
      if (kc + 1 < nk) {
        wait_vmcnt0();    // chunk kc+1 landed (chunk kc+2 is not issued yet)
        wait_lgkmcnt0();  // this wave's reads of stage kc&1 are done
        __syncthreads();
        if (kc + 2 < nk) issue(kc + 2, kc & 1);
        readk(kc + 1, 0, fa0, fb0);
      }
      mfma(fa1, fb1);
    }
  }
  const int c0 = n0 + wv * 64 + 4 * gq;
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int e = m0 + i * 16 + li;
    if (e >= Eh) continue;
    float *prow = part + ((size_t)ts * E + (size_t)h * Eh + e) * dh;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int c = c0 + f * 16;
      if (c < dh) *(f32x4 *)(prow + c) = acc[i][f];
    }
  }
}

// dbias[e] = sum_t dl[t][e] in two passes: block (64 experts, token chunk c)
// sums its chunk's rows (lane = expert: coalesced rows; wave w takes every
// fourth token, then the four waves are added in order) into part[c][e]; then
// one wave per expert adds the chunks (lane l: chunks l, l + 64, ... in order,
// then a fixed butterfly over the lanes).  The order is fixed: reproducible.
__global__ __launch_bounds__(256) void router_dbias_part_kernel(const float *__restrict__ dl, int T, int E, int per,
                                                                float *__restrict__ part) {
  __shared__ float sw[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, e = blockIdx.x * 64 + lane, c = blockIdx.y;
  const int t0 = c * per, t1 = min(T, t0 + per);
  float v = 0.f;
  if (e < E) {
#pragma unroll 4
    for (int t = t0 + w; t < t1; t += 4) v += dl[(size_t)t * E + e];
  }
  sw[w][lane] = v;
  __syncthreads();
  if (w == 0 && e < E) part[(size_t)c * E + e] = ((sw[0][lane] + sw[1][lane]) + sw[2][lane]) + sw[3][lane];
}
__global__ __launch_bounds__(256) void router_dbias_sum_kernel(const float *__restrict__ part, int E, int nch,
                                                               float *__restrict__ dbias) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (e >= E) return;  // whole waves
  float v = 0.f;
  for (int c = lane; c < nch; c += 64) v += part[(size_t)c * E + e];
  v = group_sum_fixed(v, WAVE);
  if (lane == 0) dbias[e] = v;
}

// ---------------------------------------------------------------- input gradient
// For column c of head h (c = h*dh + cl):
//   out[t][c] = [dy[t][c]] + [dxs[t][c]] + sum_{j in head h} dXr[row_of[t][j]][cl]
//               + sum_{e in head h} dl[t][e] W_r[e][cl],
// float32 in that order (the router term over experts ascending), rounded
// once: the layer's dx (one head or no latent projection), or the gradient of
// the latent u.  A block takes DX_TOK consecutive tokens and 2 * blockDim.x
// columns of one head; each thread owns two adjacent columns, so a router
// weight load of two elements feeds 2 * DX_TOK multiply-adds.  The block's dl
// rows (its head's slice) are staged in LDS once and read as broadcasts.
// Measured on the group-limited shapes (8192 tokens, 5120 columns, 160
// experts, top-6): the row gather and the router term each take about half
// of the kernel's time, the former near the HBM rate of its bytes.
constexpr int DX_TOK = 16;
template <typename T> struct Pair2;
template <> struct Pair2<uint16_t> {  // two adjacent bf16 (4-byte aligned)
  __device__ __forceinline__ static void load(const uint16_t *p, float &a, float &b) {
    const uint32_t u = *(const uint32_t *)p;
    a = bf16_to_f32((uint16_t)(u & 0xFFFFu));
    b = bf16_to_f32((uint16_t)(u >> 16));
  }
  __device__ __forceinline__ static void store(uint16_t *p, float a, float b) {
    *(uint32_t *)p = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
  }
};
template <> struct Pair2<float> {  // two adjacent float32 (8-byte aligned)
  __device__ __forceinline__ static void load(const float *p, float &a, float &b) {
    const float2 u = *(const float2 *)p;
    a = u.x;
    b = u.y;
  }
  __device__ __forceinline__ static void store(float *p, float a, float b) { *(float2 *)p = make_float2(a, b); }
};

template <typename TA, typename TR>
__global__ __launch_bounds__(256) void bwd_dx_kernel(const TA *__restrict__ dy, const TA *__restrict__ dxs,
                                                     const TA *__restrict__ dXr, const int32_t *__restrict__ row_of,
                                                     const float *__restrict__ dl, const TR *__restrict__ w_r, int T,
                                                     int D, int dh, int H, int K, int k, int E, int Eh, int residual,
                                                     TA *__restrict__ dx) {
  __shared__ float4 sdl4[DX_TOK * 64];  // [DX_TOK][EP] with EP = E_h rounded up to 4 (E_h <= 256)
  float *sdl = (float *)sdl4;
  const int EP = (Eh + 3) & ~3;
  const int ncol = 2 * blockDim.x, cpb = (dh + ncol - 1) / ncol;
  const int h = blockIdx.y / cpb, cl = (blockIdx.y % cpb) * ncol + 2 * threadIdx.x;
  const int t0 = blockIdx.x * DX_TOK;
  const int nt = min(DX_TOK, T - t0);
  for (int i = threadIdx.x; i < DX_TOK * EP; i += blockDim.x) {
    const int tt = i / EP, e = i - tt * EP;
    sdl[i] = (tt < nt && e < Eh) ? dl[(size_t)(t0 + tt) * E + (size_t)h * Eh + e] : 0.f;
  }
  __syncthreads();
  if (cl >= dh) return;  // dh is even, so cl + 1 < dh too
  const int c = h * dh + cl;
  float a0[DX_TOK], a1[DX_TOK];
#pragma unroll
  for (int i = 0; i < DX_TOK; ++i) {
    float v0 = 0.f, v1 = 0.f;
    if (i < nt) {
      const int t = t0 + i;
      const size_t o = (size_t)t * D + c;
      if (residual) Pair2<TA>::load(dy + o, v0, v1);
      if (dxs) {
        float u0, u1;
        Pair2<TA>::load(dxs + o, u0, u1);
        v0 += u0;
        v1 += u1;
      }
      for (int q = 0; q < k; ++q) {
        const int r = row_of[(size_t)t * K + h * k + q];
        if (r >= 0) {
          float u0, u1;
          Pair2<TA>::load(dXr + (size_t)r * dh + cl, u0, u1);
          v0 += u0;
          v1 += u1;
        }
      }
    }
    a0[i] = v0;
    a1[i] = v1;
  }
  const TR *wr = w_r + (size_t)h * Eh * dh + cl;
  int e = 0;
  for (; e + 4 <= Eh; e += 4) {
    float w0[4], w1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) Pair2<TR>::load(wr + (size_t)(e + u) * dh, w0[u], w1[u]);
#pragma unroll
    for (int i = 0; i < DX_TOK; ++i) {
      const float4 l = sdl4[(i * EP + e) >> 2];
      a0[i] += l.x * w0[0];
      a0[i] += l.y * w0[1];
      a0[i] += l.z * w0[2];
      a0[i] += l.w * w0[3];
      a1[i] += l.x * w1[0];
      a1[i] += l.y * w1[1];
      a1[i] += l.z * w1[2];
      a1[i] += l.w * w1[3];
    }
  }
  for (; e < Eh; ++e) {
    float w0, w1;
    Pair2<TR>::load(wr + (size_t)e * dh, w0, w1);
#pragma unroll
    for (int i = 0; i < DX_TOK; ++i) {
      const float l = sdl[i * EP + e];
      a0[i] += l * w0;
      a1[i] += l * w1;
    }
  }
#pragma unroll
  for (int i = 0; i < DX_TOK; ++i)
    if (i < nt) Pair2<TA>::store(dx + (size_t)(t0 + i) * D + c, a0[i], a1[i]);
}

// ---------------------------------------------------------------- launchers
template <typename TA>
static int transpose_t(const void *src, long ld_src, long bs_src, const int32_t *rmap, long nvalid, long njcols,
                       int ncols, int coff, void *dst, long ld_dst, long bs_dst, int batches, int kchunk,
                       hipStream_t st) {
  if (njcols <= 0 || ncols <= 0 || batches <= 0) return 0;
  if (kchunk && (njcols % 64 || ncols > ld_dst)) return -2;  // whole k-chunks, rows inside dst
  dim3 grid((unsigned)((njcols + 63) / 64), (unsigned)((ncols + 63) / 64), (unsigned)batches);
  hipLaunchKernelGGL((transpose_kernel<TA>), grid, dim3(256), 0, st, (const TA *)src, ld_src, bs_src, rmap, nvalid,
                     njcols, ncols, coff, (TA *)dst, ld_dst, bs_dst, kchunk);
  return launch_status("transpose");
}

int launch_transpose(bool f32, const void *src, long ld_src, long bs_src, const int32_t *rmap, long nvalid,
                     long njcols, int ncols, int coff, void *dst, long ld_dst, long bs_dst, int batches,
                     hipStream_t st, int kchunk) {
  return f32 ? transpose_t<float>(src, ld_src, bs_src, rmap, nvalid, njcols, ncols, coff, dst, ld_dst, bs_dst,
                                  batches, kchunk, st)
             : transpose_t<uint16_t>(src, ld_src, bs_src, rmap, nvalid, njcols, ncols, coff, dst, ld_dst, bs_dst,
                                     batches, kchunk, st);
}

int launch_bwd_rows(const Shape &s, const void *dy, long ld_dy, const void *y_perm, const float *gates,
                    const int32_t *src_of, const int32_t *topk_idx, const int32_t *offsets, void *dY, float *dg,
                    hipStream_t st) {
  const long tk = (long)s.T * s.K;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)std::min<long>((tk + 255) / 256, 4096)), dim3(256), 0, st, dg,
                     tk);
  if (int rc = launch_status("zero gate gradients")) return rc;
  if (s.R_max == 0) return 0;
  // W lanes per row: the row's 16-byte chunks (d_head is a multiple of 64), at most 64
  const int chunks = s.dh * (s.act_f32 ? 4 : 2) / 16;
  const int W = chunks >= 64 ? 64 : chunks >= 32 ? 32 : chunks >= 16 ? 16 : 8;
  const long waves = (s.R_max * W + 63) / 64;
  const dim3 grid((unsigned)((waves + 3) / 4));
  auto go = [&](auto kern, auto *typed) {
    using T = std::remove_pointer_t<decltype(typed)>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, (const T *)dy, (const T *)y_perm, gates, src_of, topk_idx,
                       offsets, s.E, s.Eh, s.K, s.dh, ld_dy, (T *)dY, dg);
  };
  if (s.act_f32) {
    if (W == 64) go(bwd_rows_kernel<float, 64>, (float *)nullptr);
    else if (W == 32) go(bwd_rows_kernel<float, 32>, (float *)nullptr);
    else go(bwd_rows_kernel<float, 16>, (float *)nullptr);  // f32 rows hold at least 16 chunks
  } else {
    if (W == 64) go(bwd_rows_kernel<uint16_t, 64>, (uint16_t *)nullptr);
    else if (W == 32) go(bwd_rows_kernel<uint16_t, 32>, (uint16_t *)nullptr);
    else if (W == 16) go(bwd_rows_kernel<uint16_t, 16>, (uint16_t *)nullptr);
    else go(bwd_rows_kernel<uint16_t, 8>, (uint16_t *)nullptr);
  }
  return launch_status("backward rows");
}

// The backward's activation step from the forward's kept pre-activations
// (the forward's SwiGLU gate g and up u, or ReLU a, rounded to the act dtype
// as the forward stored them): with the upstream dH, dA = dH u SiLU'(g) and
// dB = dH SiLU(g) (dA|dB rows of 2 d_ff), H = SiLU(g) u; ReLU: dA = dH [a > 0],
// H = max(a, 0).  The same arithmetic as the recompute GEMM's backward
// epilogue, on the kept values instead of recomputed float32 products.  One
// thread per four consecutive hidden units of a row (grid-stride; rows below
// offsets[E]).
// four consecutive elements as one 8-byte (bf16) or 16-byte (float32) access
template <typename TE> struct Four;
template <> struct Four<uint16_t> {
  __device__ __forceinline__ static void load(const uint16_t *p, float o[4]) {
    const uint2 u = *(const uint2 *)p;
    o[0] = bf16_to_f32((uint16_t)(u.x & 0xFFFFu)); o[1] = bf16_to_f32((uint16_t)(u.x >> 16));
    o[2] = bf16_to_f32((uint16_t)(u.y & 0xFFFFu)); o[3] = bf16_to_f32((uint16_t)(u.y >> 16));
  }
  __device__ __forceinline__ static void store(uint16_t *p, const float v[4]) {
    uint2 u;
    u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *(uint2 *)p = u;
  }
};
template <> struct Four<float> {
  __device__ __forceinline__ static void load(const float *p, float o[4]) {
    const float4 u = *(const float4 *)p;
    o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w;
  }
  __device__ __forceinline__ static void store(float *p, const float v[4]) {
    *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
  }
};

template <typename TE, bool GLU>
__global__ __launch_bounds__(256) void bwd_saved_act_kernel(const TE *__restrict__ gu, const TE *__restrict__ dH,
                                                            TE *__restrict__ dAB, TE *__restrict__ H,
                                                            const int32_t *__restrict__ offsets, int E, long dff) {
  const long q4 = dff / 4;  // quads per row (d_ff is a multiple of 64)
  const long total = (long)offsets[E] * q4;
  const long mg = GLU ? 2 * dff : dff;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    const long r = i / q4, c = (i - r * q4) * 4;
    float dh[4], a[4], b[4], da[4], db[4], h[4];
    Four<TE>::load(dH + r * dff + c, dh);
    Four<TE>::load(gu + r * mg + c, a);
    if constexpr (GLU) Four<TE>::load(gu + r * mg + dff + c, b);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if constexpr (GLU) {
        const float gt = a[v], up = b[v];
        const float sg = 1.0f / (1.0f + __expf(-gt)), si = gt * sg;
        da[v] = dh[v] * up * (sg * (1.0f + gt * (1.0f - sg)));
        db[v] = dh[v] * si;
        h[v] = si * up;
      } else {
        da[v] = a[v] > 0.0f ? dh[v] : 0.0f;
        h[v] = fmaxf(a[v], 0.0f);
      }
    }
    Four<TE>::store(dAB + r * mg + c, da);
    if constexpr (GLU) Four<TE>::store(dAB + r * mg + dff + c, db);
    Four<TE>::store(H + r * dff + c, h);
  }
}

int launch_bwd_saved_act(const Shape &s, const void *gu, const void *dH, void *dAB, void *H, const int32_t *offsets,
                         hipStream_t st) {
  if (s.R_max == 0) return 0;
  const long total = s.R_max * (long)s.dff / 4;
  const unsigned grid = (unsigned)std::min<long>((total + 255) / 256, 16384);
  const bool glu = s.act == 1;
  if (s.act_f32) {
    if (glu) hipLaunchKernelGGL((bwd_saved_act_kernel<float, true>), dim3(grid), dim3(256), 0, st, (const float *)gu,
                                (const float *)dH, (float *)dAB, (float *)H, offsets, s.E, (long)s.dff);
    else hipLaunchKernelGGL((bwd_saved_act_kernel<float, false>), dim3(grid), dim3(256), 0, st, (const float *)gu,
                            (const float *)dH, (float *)dAB, (float *)H, offsets, s.E, (long)s.dff);
  } else {
    if (glu) hipLaunchKernelGGL((bwd_saved_act_kernel<uint16_t, true>), dim3(grid), dim3(256), 0, st,
                                (const uint16_t *)gu, (const uint16_t *)dH, (uint16_t *)dAB, (uint16_t *)H, offsets,
                                s.E, (long)s.dff);
    else hipLaunchKernelGGL((bwd_saved_act_kernel<uint16_t, false>), dim3(grid), dim3(256), 0, st,
                            (const uint16_t *)gu, (const uint16_t *)dH, (uint16_t *)dAB, (uint16_t *)H, offsets,
                            s.E, (long)s.dff);
  }
  return launch_status("backward activation from kept pre-activations");
}

int launch_bwd_pad(const Shape &s, const int32_t *offsets, const int32_t *src_of, int32_t *poff, int32_t *pmap_r,
                   int32_t *pmap_x, long npad, hipStream_t st) {
  hipLaunchKernelGGL(bwd_poff_kernel, dim3(1), dim3(1024), 0, st, offsets, s.E, poff);
  if (int rc = launch_status("expert padding")) return rc;
  if (npad <= 0) return 0;
  hipLaunchKernelGGL(bwd_pmap_kernel, dim3((unsigned)std::min<long>((npad + 255) / 256, 8192)), dim3(256), 0, st,
                     offsets, poff, src_of, s.E, s.Eh, s.H, s.K, npad, pmap_r, pmap_x);
  return launch_status("padding map");
}

// seq_cnt[s][e] by integer LDS atomics (order-free), one block per sequence
__global__ __launch_bounds__(256) void seq_counts_kernel(const int32_t *__restrict__ topk_idx, int E, int K, int L,
                                                         int32_t *__restrict__ seq_cnt) {
  extern __shared__ int cnt[];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const long a0 = (long)blockIdx.x * L * K;
  for (long i = tid; i < (long)L * K; i += 256) atomicAdd(&cnt[topk_idx[a0 + i]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 256) seq_cnt[(size_t)blockIdx.x * E + e] = cnt[e];
}

int launch_seq_counts(const Shape &s, const int32_t *topk_idx, int32_t *seq_cnt, hipStream_t st) {
  hipLaunchKernelGGL(seq_counts_kernel, dim3((unsigned)(s.T / s.seq_len)), dim3(256), (size_t)s.E * 4, st, topk_idx,
                     s.E, s.K, s.seq_len, seq_cnt);
  return launch_status("sequence counts");
}

int launch_router_bwd(const Shape &s, const float *logits, const int32_t *topk_idx, const float *gates,
                      const float *dg, const int32_t *demand, float lam, const int32_t *seq_cnt, float seq_w,
                      const void *x, float *dl, uint16_t *planes, float *part, float *dw_router, float *dbias,
                      hipStream_t st) {
  const long pairs = (long)s.T * s.H;
  if (pairs > 0) {
    const int L = s.seq_len > 0 ? s.seq_len : 1;
    auto go = [&](auto kern, int w) {
      const long waves = (pairs * w + 63) / 64;
      hipLaunchKernelGGL(kern, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, logits, topk_idx, gates, dg,
                         demand, s.T, s.H, s.E, s.Eh, s.K, s.k, s.renorm, lam, seq_cnt, L, seq_w, dl);
    };
    if (s.Eh <= 8) go(router_bwd_kernel<8>, 8);
    else if (s.Eh <= 16) go(router_bwd_kernel<16>, 16);
    else if (s.Eh <= 32) go(router_bwd_kernel<32>, 32);
    else go(router_bwd_kernel<64>, 64);
    if (int rc = launch_status("router backward")) return rc;
  }
  if (dbias) {
    // partials in `part` (at least ROUTER_DBIAS_CHUNKS * E floats; the weight
    // gradient overwrites them afterwards, in stream order)
    const int per = (int)std::max<long>(16, ((long)s.T + ROUTER_DBIAS_CHUNKS - 1) / ROUTER_DBIAS_CHUNKS);
    const int nch = (int)std::max<long>(1, ((long)s.T + per - 1) / per);
    hipLaunchKernelGGL(router_dbias_part_kernel, dim3((unsigned)((s.E + 63) / 64), (unsigned)nch), dim3(256), 0, st,
                       dl, s.T, s.E, per, part);
    if (int rc = launch_status("router bias gradient")) return rc;
    hipLaunchKernelGGL(router_dbias_sum_kernel, dim3((unsigned)((s.E + 3) / 4)), dim3(256), 0, st, part, s.E,
                       nch, dbias);
    if (int rc = launch_status("router bias gradient")) return rc;
  }
  const long ldx = (long)s.H * s.dh, n = (long)s.E * s.dh;
  int nsplit;
  if (s.act_f32) {
    nsplit = router_wgrad_split(s);
    const dim3 grid((unsigned)((s.Eh + 63) / 64), (unsigned)((s.dh + 63) / 64), (unsigned)(nsplit * s.H));
    hipLaunchKernelGGL((router_wgrad_kernel<float>), grid, dim3(256), 0, st, dl, (const float *)x, ldx, s.T, s.E,
                       s.Eh, s.dh, nsplit, part);
  } else {
    const RouterWgradGeom g = router_wgrad_geom(s);
    nsplit = g.nsplit;
    if (g.tp > 0) {
      const dim3 pg((unsigned)(g.tp / 64), (unsigned)((g.ep + 63) / 64), (unsigned)s.H);
      hipLaunchKernelGGL(router_dl_planes_kernel, pg, dim3(256), 0, st, dl, s.T, s.E, s.Eh, g.ep, g.tp, planes);
      if (int rc = launch_status("router gradient planes")) return rc;
    }
    float *out = nsplit == 1 ? dw_router : part;
    const unsigned blocks = (unsigned)((long)(g.ep / g.bm) * ((s.dh + 255) / 256) * nsplit * s.H);
    const size_t lds = (size_t)2 * 3 * g.bm * 8 * 16 + 2 * RW_BSTAGE;
    const uint16_t *xb = (const uint16_t *)x;
    if (g.bm == 16)
      hipLaunchKernelGGL((router_wgrad_mfma_kernel<16>), dim3(blocks), dim3(256), lds, st, planes, xb, ldx, s.T,
                         g.tp, s.E, s.Eh, g.ep, s.dh, s.H, g.per, nsplit, out);
    else if (g.bm == 32)
      hipLaunchKernelGGL((router_wgrad_mfma_kernel<32>), dim3(blocks), dim3(256), lds, st, planes, xb, ldx, s.T,
                         g.tp, s.E, s.Eh, g.ep, s.dh, s.H, g.per, nsplit, out);
    else
      hipLaunchKernelGGL((router_wgrad_mfma_kernel<64>), dim3(blocks), dim3(256), lds, st, planes, xb, ldx, s.T,
                         g.tp, s.E, s.Eh, g.ep, s.dh, s.H, g.per, nsplit, out);
    if (nsplit == 1) return launch_status("router weight gradient");
  }
  if (int rc = launch_status("router weight gradient")) return rc;
  hipLaunchKernelGGL(router_wgrad_sum_kernel, dim3((unsigned)std::min<long>((n / 4 + 63) / 64, 8192)), dim3(64), 0,
                     st, part, n, nsplit, dw_router);
  return launch_status("router weight gradient");
}

__global__ void set_kwin_kernel(int32_t *kwin, int tpad, int nsplit) {
  const int s = threadIdx.x;
  if (s <= nsplit) kwin[s] = min(tpad, (int)(((long)s * tpad / nsplit + 63) / 64 * 64));
}

int launch_set_kwin(int32_t *kwin, int tpad, int nsplit, hipStream_t st) {
  hipLaunchKernelGGL(set_kwin_kernel, dim3(1), dim3(64), 0, st, kwin, tpad, nsplit);
  return launch_status("k window");
}

int launch_bwd_dx(const Shape &s, const void *dy, const void *dxs, const void *dXr, const int32_t *row_of,
                  const float *dl, const void *w_router, int residual, void *dx, hipStream_t st) {
  if (s.T == 0) return 0;
  // two columns per thread: 256 threads for heads of 512 columns or more, fewer for narrow heads
  const int nthr = std::min(256, (s.dh / 2 + 63) / 64 * 64);
  const dim3 grid((unsigned)((s.T + DX_TOK - 1) / DX_TOK), (unsigned)(s.H * ((s.dh + 2 * nthr - 1) / (2 * nthr))));
  const int D = s.H * s.dh;
  if (s.act_f32) {
    hipLaunchKernelGGL((bwd_dx_kernel<float, float>), grid, dim3(nthr), 0, st, (const float *)dy, (const float *)dxs,
                       (const float *)dXr, row_of, dl, (const float *)w_router, s.T, D, s.dh, s.H, s.K, s.k, s.E,
                       s.Eh, residual, (float *)dx);
  } else if (s.router_f32) {
    hipLaunchKernelGGL((bwd_dx_kernel<uint16_t, float>), grid, dim3(nthr), 0, st, (const uint16_t *)dy,
                       (const uint16_t *)dxs, (const uint16_t *)dXr, row_of, dl, (const float *)w_router, s.T, D,
                       s.dh, s.H, s.K, s.k, s.E, s.Eh, residual, (uint16_t *)dx);
  } else {
    hipLaunchKernelGGL((bwd_dx_kernel<uint16_t, uint16_t>), grid, dim3(nthr), 0, st, (const uint16_t *)dy,
                       (const uint16_t *)dxs, (const uint16_t *)dXr, row_of, dl, (const uint16_t *)w_router, s.T,
                       D, s.dh, s.H, s.K, s.k, s.E, s.Eh, residual, (uint16_t *)dx);
  }
  return launch_status("input gradient");
}

}  // namespace moe

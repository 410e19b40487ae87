// Dispatch: keep rule and the permutation into an expert-contiguous buffer.
//
// Capacity C with overflow through the residual: "MoE技术演进", "GShard" item 1.
// Keep the best 90 % of each expert's tokens by affinity: "MoE技术演进",
// "DeepSeek-V2" item 5 (here per expert, affinity = gate).  No dropping:
// "DeepSeek-V3" item 5.  Count tokens per expert first, then fill each
// expert's buffer: "大语言模型并行策略（七）：专家并行", "MoE 中的 all-to-all 通信".
//
// Pipeline (flat assignment a = t*K + j, chunks of CH consecutive a):
//   hist      per-chunk expert histogram (LDS integer atomics: order-free)
//   scan      per-expert prefix over chunks -> chunk bases; demand; keep rule
//             -> counts; offsets = exclusive scan of counts
//   rank      stable rank of every a among the earlier a of its expert, from
//             the chunk base + per-wave prefix + in-wave ballot match; writes
//             row_of / src_of (NONE, CAPACITY) or the expert-sorted segment
//             list (AFFINITY)
//   affinity  one block per expert: radix select of the keep-th largest gate,
//             then two ordered scans -> row_of / src_of
//   scatter   row r <- x[src_of[r] / K] (head slice), 16-byte copies
// Every count is an integer and every order is fixed by a, so the result is
// bit-reproducible.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int CH = 4096;  // assignments per chunk (256 threads x 16)

__global__ __launch_bounds__(256) void disp_hist_kernel(const int32_t *__restrict__ idx, long n, int E,
                                                        int32_t *__restrict__ hist) {
  extern __shared__ int32_t h[];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  long a0 = (long)blockIdx.x * CH;
  for (int i = threadIdx.x; i < CH; i += 256) {
    long a = a0 + i;
    if (a < n) atomicAdd(&h[idx[a]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(long)blockIdx.x * E + e] = h[e];
}

// one block of 1024 threads; E <= 1024
__global__ __launch_bounds__(1024) void disp_scan_kernel(
    int32_t *__restrict__ hist /* in: counts, out: chunk bases */, int nchunks, int E, int drop, int C,
    int keep_num, int keep_den, int32_t *__restrict__ demand, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ all_off) {
  __shared__ int32_t sc[1024];
  __shared__ int32_t sd[1024];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) {
      int v = hist[(long)c * E + e];
      hist[(long)c * E + e] = run;
      run += v;
    }
  }
  int cnt = 0;
  if (e < E) {
    if (drop == 0) cnt = run;
    else if (drop == 1) cnt = min(run, C);
    else cnt = (int)(((long)keep_num * run + keep_den - 1) / keep_den);
    demand[e] = run;
    counts[e] = cnt;
  }
  sc[e] = (e < E) ? cnt : 0;
  sd[e] = (e < E) ? run : 0;
  __syncthreads();
  // Hillis-Steele inclusive scans (integers: exact)
  for (int o = 1; o < 1024; o <<= 1) {
    int v1 = (e >= o) ? sc[e - o] : 0;
    int v2 = (e >= o) ? sd[e - o] : 0;
    __syncthreads();
    sc[e] += v1;
    sd[e] += v2;
    __syncthreads();
  }
  if (e < E) {
    offsets[e] = sc[e] - cnt;
    if (all_off) all_off[e] = sd[e] - run;
  }
  if (e == 0) {
    offsets[E] = sc[1023];
    if (all_off) all_off[E] = sd[1023];
  }
}

// lanes of this wave holding the same expert id (E <= 1024 -> 10 bits)
__device__ __forceinline__ uint64_t match_mask(int e, bool active) {
  uint64_t m = __ballot(active);
#pragma unroll
  for (int b = 0; b < 10; ++b) {
    uint64_t bal = __ballot(active && ((e >> b) & 1));
    m &= ((e >> b) & 1) ? bal : ~bal;
  }
  return active ? m : 0ull;
}

// block 256 = 4 waves per chunk; wave w owns a in [a0 + w*CH/4, a0 + (w+1)*CH/4)
__global__ __launch_bounds__(256) void disp_rank_kernel(
    const int32_t *__restrict__ idx, long n, int E, const int32_t *__restrict__ base,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ all_off, int drop, int C,
    int32_t *__restrict__ row_of, int32_t *__restrict__ src_of, int32_t *__restrict__ seg) {
  extern __shared__ int32_t cnt[];  // [4][E]: per-wave counts, then running counters
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int SUB = CH / 4;
  const long a0 = (long)blockIdx.x * CH + (long)w * SUB;
  for (int i = tid; i < 4 * E; i += 256) cnt[i] = 0;
  __syncthreads();
  for (int i = lane; i < SUB; i += 64) {
    long a = a0 + i;
    if (a < n) atomicAdd(&cnt[w * E + idx[a]], 1);
  }
  __syncthreads();
  // exclusive prefix over waves, plus the chunk base
  for (int e = tid; e < E; e += 256) {
    int run = base[(long)blockIdx.x * E + e];
    for (int q = 0; q < 4; ++q) {
      int v = cnt[q * E + e];
      cnt[q * E + e] = run;
      run += v;
    }
  }
  __syncthreads();
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i0 = 0; i0 < SUB; i0 += 64) {
    long a = a0 + i0 + lane;
    bool act = a < n;
    int e = act ? idx[a] : 0;
    uint64_t m = match_mask(e, act);
    int before = __popcll(m & lt);
    int rank = 0;
    if (act) rank = cnt[w * E + e] + before;
    // the highest lane of each group advances the counter (after every lane read it)
    bool leader = act && ((m >> lane) >> 1) == 0ull;
    if (leader) cnt[w * E + e] = rank + 1;
    if (act) {
      if (drop == 2) {
        seg[all_off[e] + rank] = (int32_t)a;
      } else {
        bool kept = (drop == 0) || rank < C;
        int row = kept ? offsets[e] + rank : -1;
        row_of[a] = row;
        if (kept) src_of[row] = (int32_t)a;
      }
    }
  }
}

// ---------------------------------------------------------------- affinity keep (per expert block)
__device__ __forceinline__ int block_excl_scan(int v, int *tmp, int *total) {
  // 256 threads, fixed order
  const int tid = threadIdx.x;
  tmp[tid] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    int u = (tid >= o) ? tmp[tid - o] : 0;
    __syncthreads();
    tmp[tid] += u;
    __syncthreads();
  }
  int incl = tmp[tid];
  *total = tmp[255];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(256) void disp_affinity_kernel(
    const int32_t *__restrict__ seg, const int32_t *__restrict__ all_off, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, const float *__restrict__ topk_w, int32_t *__restrict__ row_of,
    int32_t *__restrict__ src_of) {
  __shared__ int hist[256];
  __shared__ int tmp[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  const int e = blockIdx.x, tid = threadIdx.x;
  const int beg = all_off[e], n = all_off[e + 1] - beg;
  const int keep = counts[e];
  const int out0 = offsets[e];
  if (n == 0) return;
  // threshold key: the keep-th largest gate bit pattern (gates are >= 0, so
  // their float bits order like the values)
  uint32_t prefix = 0, pmask = 0;
  int need = keep;  // how many still to take from keys matching prefix
  if (keep < n) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += 256) {
        uint32_t key = __float_as_uint(topk_w[seg[beg + i]]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
      }
      __syncthreads();
      if (tid == 0) {
        int acc = 0, d = 255;
        for (; d > 0; --d) {
          if (acc + hist[d] >= need) break;
          acc += hist[d];
        }
        s_prefix = prefix | ((uint32_t)d << shift);
        s_need = need - acc;
      }
      __syncthreads();
      prefix = s_prefix;
      need = s_need;
      pmask |= 255u << shift;
      __syncthreads();
    }
  }
  // kept iff key > thr, or key == thr and among the first `need` equal keys (by a)
  int eq_seen = 0, kept_seen = 0;
  for (int i0 = 0; i0 < n; i0 += 256) {
    int i = i0 + tid;
    bool act = i < n;
    int a = act ? seg[beg + i] : 0;
    uint32_t key = act ? __float_as_uint(topk_w[a]) : 0u;
    bool kept;
    int tot;
    if (keep >= n) {
      kept = act;
    } else {
      bool eq = act && key == prefix;
      int eq_before = block_excl_scan(eq ? 1 : 0, tmp, &tot);
      kept = act && (key > prefix || (eq && eq_seen + eq_before < need));
      eq_seen += tot;
    }
    int kb = block_excl_scan(kept ? 1 : 0, tmp, &tot);
    if (act) {
      // never past this expert's `keep` rows, even if the selection were off
      kept = kept && (kept_seen + kb < keep);
      int row = kept ? out0 + kept_seen + kb : -1;
      row_of[a] = row;
      if (kept) src_of[row] = a;
    }
    kept_seen += tot;
  }
}

// ---------------------------------------------------------------- row gather
template <typename TA>
__global__ __launch_bounds__(256) void disp_scatter_kernel(
    const TA *__restrict__ x, const int32_t *__restrict__ src_of, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ offsets, TA *__restrict__ x_perm, int E, int K, int Eh, int dh, int ldx,
    int rows_per_block, long n_assign) {
  const int R = offsets[E];
  const long r0 = (long)blockIdx.x * rows_per_block;
  if (r0 >= R) return;
  const int nrows = (int)min((long)rows_per_block, (long)R - r0);
  const int cpr = dh * (int)sizeof(TA) / 16;  // 16-byte chunks per row
  const int total = nrows * cpr;
  for (int i = threadIdx.x; i < total; i += 256) {
    int rr = i / cpr, q = i - rr * cpr;
    long r = r0 + rr;
    int a = src_of[r];
    if (a < 0 || a >= n_assign) continue;  // defensive: rows are always written
    int t = a / K;
    int h = idx[a] / Eh;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (size_t)t * ldx + (size_t)h * dh);
    u32x4 *dst = reinterpret_cast<u32x4 *>(x_perm + (size_t)r * dh);
    dst[q] = src[q];
  }
}

// ---------------------------------------------------------------- host
static long n_chunks(const Shape &s) { return ((long)s.T * s.K + CH - 1) / CH; }

size_t dispatch_ws_bytes(const Shape &s) {
  size_t b = align_up((size_t)n_chunks(s) * s.E * 4, 256);  // chunk hist / bases
  b += align_up((size_t)(s.E + 1) * 4, 256);                  // all_off
  if (s.drop == 2) b += align_up((size_t)s.T * s.K * 4, 256);  // expert-sorted segments
  return b;
}

int launch_dispatch(const Shape &s, const int32_t *topk_idx, const float *topk_w, const void *x,
                    int32_t *demand, int32_t *counts, int32_t *offsets, int32_t *row_of, int32_t *src_of,
                    void *x_perm, void *ws, hipStream_t st) {
  const long n = (long)s.T * s.K;
  const long nc = n_chunks(s);
  char *p = (char *)ws;
  int32_t *hist = (int32_t *)p;
  p += align_up((size_t)nc * s.E * 4, 256);
  int32_t *all_off = (int32_t *)p;
  p += align_up((size_t)(s.E + 1) * 4, 256);
  int32_t *seg = (s.drop == 2) ? (int32_t *)p : nullptr;

  hipLaunchKernelGGL(disp_hist_kernel, dim3(nc), dim3(256), s.E * 4, st, topk_idx, n, s.E, hist);
  if (hipGetLastError() != hipSuccess) return -4;
  hipLaunchKernelGGL(disp_scan_kernel, dim3(1), dim3(1024), 0, st, hist, (int)nc, s.E, s.drop, s.C,
                     s.keep_num, s.keep_den, demand, counts, offsets, s.drop == 2 ? all_off : nullptr);
  if (hipGetLastError() != hipSuccess) return -4;
  hipLaunchKernelGGL(disp_rank_kernel, dim3(nc), dim3(256), 4 * s.E * 4, st, topk_idx, n, s.E, hist,
                     offsets, all_off, s.drop, s.C, row_of, src_of, seg);
  if (hipGetLastError() != hipSuccess) return -4;
  if (s.drop == 2) {
    hipLaunchKernelGGL(disp_affinity_kernel, dim3(s.E), dim3(256), 0, st, seg, all_off, counts, offsets,
                       topk_w, row_of, src_of);
    if (hipGetLastError() != hipSuccess) return -4;
  }
  const int esz = s.act_f32 ? 4 : 2;
  long rpb_ = 32768 / ((long)s.dh * esz);
  int rpb = rpb_ < 1 ? 1 : (int)rpb_;
  long blocks = (s.R_max + rpb - 1) / rpb;
  if (blocks > 0) {
    if (s.act_f32)
      hipLaunchKernelGGL(disp_scatter_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float *)x, src_of,
                         topk_idx, offsets, (float *)x_perm, s.E, s.K, s.Eh, s.dh, s.H * s.dh, rpb, n);
    else
      hipLaunchKernelGGL(disp_scatter_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st, (const uint16_t *)x,
                         src_of, topk_idx, offsets, (uint16_t *)x_perm, s.E, s.K, s.Eh, s.dh, s.H * s.dh, rpb, n);
    if (hipGetLastError() != hipSuccess) return -4;
  }
  return 0;
}

}  // namespace moe

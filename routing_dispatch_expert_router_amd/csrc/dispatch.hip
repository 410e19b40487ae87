// Dispatch: keep rule and the permutation into an expert-contiguous buffer.
//
// Capacity C with overflow through the residual: "MoE技术演进", "GShard" item 1.
// Expert choice (each expert keeps its top-C tokens): the LocMoE+ article's
// router-taxonomy paragraph; it runs as the affinity path with C as the count.
// Keep the best 90 % of each expert's tokens by affinity: "MoE技术演进",
// "DeepSeek-V2" item 5 (here per expert, affinity = gate).  No dropping:
// "DeepSeek-V3" item 5.  Count tokens per expert first, then fill each
// expert's buffer: "大语言模型并行策略（七）：专家并行", "MoE 中的 all-to-all 通信".
//
// Pipeline (flat assignment a = t*K + j, chunks of CH consecutive a):
//   hist      per-chunk expert histogram (LDS integer atomics: order-free)
//   rank      each chunk's block sums the earlier chunks' histograms (its base
//             per expert), applies the keep rule to the demand and scans the
//             kept counts into offsets (block 0 writes demand, counts,
//             offsets); then the stable rank of every a among the earlier a of
//             its expert = chunk base + per-wave prefix + in-wave ballot
//             match; writes row_of / src_of (NONE, CAPACITY) or the
//             expert-sorted segment list (AFFINITY)
//   affinity  one block per expert: radix select of the keep-th largest gate,
//             then two ordered scans -> row_of / src_of
//   scatter   token-major copy: each 16 bytes of x are read once and stored
//             to every kept row of their token (head slice)
// Every count is an integer and every order is fixed by a, so the result is
// bit-reproducible.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace moe {

// ---------------------------------------------------------------- library-held scratch
// The dispatch scratch of the workspace-free entry point: one array per GPU,
// held until the process ends.  Its name is a host-side stand-in for the
// device array; host code uses only the address hipGetSymbolAddress returns
// for the current device.
static __device__ __align__(256) unsigned char scratch[DISPATCH_SCRATCH_MAX];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // per device: the device address of `scratch`, or NULL before first use
}  // namespace

int dispatch_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -4;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return -4;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

constexpr int CH = 1024;  // assignments per chunk (256 threads x 4)

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

// exclusive scan of v[0..E) by a 256-thread block (E <= 1024, 4 per thread),
// in integers and a fixed order; returns the total
__device__ int block_scan_experts(const int *v, int *out, int E, int *tmp) {
  const int tid = threadIdx.x;
  int loc[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    loc[i] = e < E ? v[e] : 0;
    sum += loc[i];
  }
  tmp[tid] = sum;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    int u = tid >= o ? tmp[tid - o] : 0;
    __syncthreads();
    tmp[tid] += u;
    __syncthreads();
  }
  int run = tmp[tid] - sum;
  const int total = tmp[255];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    if (e < E) out[e] = run;
    run += loc[i];
  }
  __syncthreads();
  return total;
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

// One block (4 waves) per chunk; wave w owns a in [a0 + w*CH/4, a0 + (w+1)*CH/4).
__global__ __launch_bounds__(256) void disp_rank_kernel(
    const int32_t *__restrict__ idx, long n, int E, int nchunks, const int32_t *__restrict__ hist, int drop,
    int C, int keep_num, int keep_den, int32_t *__restrict__ demand, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ all_off_out, int32_t *__restrict__ row_of,
    int32_t *__restrict__ src_of, int32_t *__restrict__ seg) {
  extern __shared__ int32_t sm[];
  int32_t *cnt = sm;            // [4][E] per-wave counts, then running ranks
  int32_t *base = sm + 4 * E;   // [E] this chunk's base per expert
  int32_t *dem = base + E;      // [E] demand
  int32_t *kept = dem + E;      // [E] kept counts
  int32_t *off = kept + E;      // [E] first row of each expert
  int32_t *aoff = off + E;      // [E] first slot of each expert in the affinity segments
  __shared__ int tmp[256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = blockIdx.x;
  for (int e = tid; e < E; e += 256) {
    int b = 0, tot = 0;
#pragma unroll 8
    for (int q = 0; q < nchunks; ++q) {
      const int v = hist[(long)q * E + e];
      b += q < c ? v : 0;
      tot += v;
    }
    base[e] = b;
    dem[e] = tot;
    kept[e] = drop == DROP_NONE       ? tot
              : drop == DROP_AFFINITY ? (int)(((long)keep_num * tot + keep_den - 1) / keep_den)
                                      : min(tot, C);  // capacity, or the experts' top-C choice
  }
  __syncthreads();
  const int R = block_scan_experts(kept, off, E, tmp);
  if (drop >= DROP_AFFINITY) block_scan_experts(dem, aoff, E, tmp);
  if (c == 0) {
    for (int e = tid; e < E; e += 256) {
      demand[e] = dem[e];
      counts[e] = kept[e];
      offsets[e] = off[e];
      if (drop >= DROP_AFFINITY) all_off_out[e] = aoff[e];
    }
    if (tid == 0) {
      offsets[E] = R;
      if (drop >= DROP_AFFINITY) all_off_out[E] = (int)n;
    }
  }
  constexpr int SUB = CH / 4;
  const long a0 = (long)c * CH + (long)w * SUB;
  for (int i = tid; i < 4 * E; i += 256) cnt[i] = 0;
  __syncthreads();
  for (int i = lane; i < SUB; i += 64) {
    long a = a0 + i;
    if (a < n) atomicAdd(&cnt[w * E + idx[a]], 1);
  }
  __syncthreads();
  // exclusive prefix over the block's waves, plus the chunk base
  for (int e = tid; e < E; e += 256) {
    int run = base[e];
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
      if (drop >= DROP_AFFINITY) {
        seg[aoff[e] + rank] = (int32_t)a;
      } else {
        bool kp = (drop == DROP_NONE) || rank < C;
        int row = kp ? off[e] + rank : -1;
        row_of[a] = row;
        if (kp) src_of[row] = (int32_t)a;
      }
    }
  }
}

// ---------------------------------------------------------------- affinity keep (per expert block)
// Exclusive scan of the values of the block's first 256 threads (fixed
// order); every thread of the block takes part in the barriers.
__device__ __forceinline__ int block_excl_scan(int v, int *tmp, int *total) {
  const int tid = threadIdx.x;
  const bool own = tid < 256;
  if (own) tmp[tid] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    int u = (own && tid >= o) ? tmp[tid - o] : 0;
    __syncthreads();
    if (own) tmp[tid] += u;
    __syncthreads();
  }
  int incl = own ? tmp[tid] : v;
  *total = tmp[255];
  __syncthreads();
  return incl - v;
}

// Exclusive count of set flags over an NT-thread block (thread order) and the
// total: in-wave ballot prefix plus the earlier waves' counts.
template <int NT>
__device__ __forceinline__ int block_excl_count(bool f, int *wsum, int *total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t b = __ballot(f);
  const int in_wave = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[w] = __popcll(b);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int q = 0; q < NT / 64; ++q) {
    const int v = wsum[q];
    before += q < w ? v : 0;
    tot += v;
  }
  __syncthreads();  // wsum is rewritten by the next call
  *total = tot;
  return before + in_wave;
}

// One block of NT threads per expert (1024 when experts hold many
// assignments, as with expert choice, else 256).  The expert's gate keys and
// assignments (up to `cap` of them, in dynamic LDS) are staged once; a 4-pass radix select (8 bits per
// pass, digit found by a suffix scan over the 256 bins) gives the keep-th
// largest key; two ordered scans then pick the kept assignments and their rows.
// An expert with more than `cap` assignments reads them from global memory.
constexpr int AFF_LDS_MAX = (160 * 1024 - 4096) / 8;  // keys + indices beside ~2 KiB of static LDS

template <int NT>
__global__ __launch_bounds__(NT) void disp_affinity_kernel(
    const int32_t *__restrict__ seg, const int32_t *__restrict__ all_off, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, const float *__restrict__ topk_w, int32_t *__restrict__ row_of,
    int32_t *__restrict__ src_of, int cap, int ecE) {
  extern __shared__ uint32_t dyn_lds[];
  uint32_t *skey = dyn_lds;
  int *sa = (int *)(dyn_lds + cap);
  __shared__ int hist[256];
  __shared__ int tmp[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  const int e = blockIdx.x, tid = threadIdx.x;
  const int beg = all_off[e], n = all_off[e + 1] - beg;
  const int keep = counts[e];
  const int out0 = offsets[e];
  if (n == 0) return;
  // the expert's i-th assignment in flat order: from the expert-sorted
  // segments, or (expert choice, ecE = E) token i's slot e, a = i * E + e
  auto a_src = [&](int i) -> int { return ecE ? i * ecE + e : seg[beg + i]; };
  if (keep == 0) {  // nothing kept (capacity 0): every assignment of e is dropped
    for (int i = tid; i < n; i += NT) row_of[a_src(i)] = -1;
    return;
  }
  const bool staged = n <= cap;
  if (staged) {
    for (int i = tid; i < n; i += NT) {
      const int a = a_src(i);
      sa[i] = a;
      skey[i] = __float_as_uint(topk_w[a]);  // gates are >= 0: their bits order like the values
    }
    __syncthreads();
  }
  auto key_of = [&](int i) -> uint32_t { return staged ? skey[i] : __float_as_uint(topk_w[a_src(i)]); };
  auto a_of = [&](int i) -> int { return staged ? sa[i] : a_src(i); };
  uint32_t prefix = 0, pmask = 0;
  int need = keep;  // how many keys still to take among those matching prefix
  if (keep < n) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += NT) {
        const uint32_t key = key_of(i);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
      }
      __syncthreads();
      // thread t looks at digit d = 255 - t; `above` = keys with a larger digit
      const int d = 255 - tid;
      const int v = tid < 256 ? hist[d] : 0;
      int tot;
      const int above = block_excl_scan(v, tmp, &tot);
      if (tid < 256 && above < need && above + v >= need) {
        s_prefix = prefix | ((uint32_t)d << shift);
        s_need = need - above;
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
  for (int i0 = 0; i0 < n; i0 += NT) {
    const int i = i0 + tid;
    const bool act = i < n;
    const int a = act ? a_of(i) : 0;
    const uint32_t key = act ? key_of(i) : 0u;
    bool kept;
    int tot;
    if (keep >= n) {
      kept = act;
    } else {
      const bool eq = act && key == prefix;
      const int eq_before = block_excl_count<NT>(eq, tmp, &tot);
      kept = act && (key > prefix || (eq && eq_seen + eq_before < need));
      eq_seen += tot;
    }
    const int kb = block_excl_count<NT>(kept, tmp, &tot);
    if (act) {
      // never past this expert's `keep` rows, even if the selection were off
      kept = kept && (kept_seen + kb < keep);
      const int row = kept ? out0 + kept_seen + kb : -1;
      row_of[a] = row;
      if (kept) src_of[row] = a;
    }
    kept_seen += tot;
  }
}

// Expert choice: every token offers one slot to every expert, so expert e's
// assignments are a = t * E + e for t = 0..T-1, already in flat order:
// demand T, kept min(C, T), offsets in closed form.  One block.
__global__ __launch_bounds__(256) void disp_ec_counts_kernel(int E, int T, int C, int32_t *__restrict__ demand,
                                                             int32_t *__restrict__ counts,
                                                             int32_t *__restrict__ offsets,
                                                             int32_t *__restrict__ all_off) {
  const int kept = min(C, T);
  for (int e = threadIdx.x; e <= E; e += 256) {
    if (e < E) {
      demand[e] = T;
      counts[e] = kept;
    }
    offsets[e] = e * kept;
    all_off[e] = e * T;
  }
}

// ---------------------------------------------------------------- row copy (token-major)
// One thread per 16 bytes of a token's row (grid-stride): read once, stored to
// every kept row of the token's head.
template <typename TA, int KH>
__global__ __launch_bounds__(256) void disp_scatter_kernel(
    const TA *__restrict__ x, const int32_t *__restrict__ row_of, TA *__restrict__ x_perm, int T, int H, int k,
    int dh, long r_max) {
  constexpr int EPC = 16 / sizeof(TA);
  const int width = H * dh;
  const int cpr = width / EPC;
  const int K = H * k;
  const long total = (long)T * cpr;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    const long t = i / cpr;
    const int q = (int)(i - t * cpr);
    const int c0 = q * EPC;
    const int h = c0 / dh;
    const u32x4 v = reinterpret_cast<const u32x4 *>(x + (size_t)t * width)[q];
    if constexpr (KH == 0) {  // many slots per token (expert choice): a plain loop
      for (int j = 0; j < k; ++j) {
        const int r = row_of[t * K + h * k + j];
        if (r >= 0 && r < r_max) reinterpret_cast<u32x4 *>(x_perm + (size_t)r * dh + (c0 - h * dh))[0] = v;
      }
    } else {
      int row[KH];
#pragma unroll
      for (int j = 0; j < KH; ++j) row[j] = j < k ? row_of[t * K + h * k + j] : -1;
#pragma unroll
      for (int j = 0; j < KH; ++j)
        if (row[j] >= 0 && row[j] < r_max)
          reinterpret_cast<u32x4 *>(x_perm + (size_t)row[j] * dh + (c0 - h * dh))[0] = v;
    }
  }
}

// ---------------------------------------------------------------- checked mode
// Validation of caller-supplied routing (moe_check_topk): one block counts the
// slots whose expert lies outside its head's range [h*E_h, (h+1)*E_h) and the
// slots that repeat an expert an earlier slot of the same token and head
// already named (expert choice: slot j of every token must be expert j), and
// writes the count; no atomics on global memory, no initial value needed.
__global__ __launch_bounds__(1024) void topk_check_kernel(const int32_t *__restrict__ idx, int T, int H, int k,
                                                          int Eh, int all_experts, int32_t *__restrict__ status) {
  __shared__ int part[1024];
  const int K = H * k;
  int bad = 0;
  for (long t = threadIdx.x; t < T; t += 1024) {
    const int32_t *row = idx + t * K;
    for (int h = 0; h < H; ++h) {
      for (int j = 0; j < k; ++j) {
        const int e = row[h * k + j];
        if (all_experts) {
          bad += e != h * k + j;
          continue;
        }
        bool b = e < h * Eh || e >= (h + 1) * Eh;
        for (int i = 0; i < j && !b; ++i) b = row[h * k + i] == e;
        bad += b;
      }
    }
  }
  part[threadIdx.x] = bad;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *status = part[0];
}

int launch_topk_check(const Shape &s, const int32_t *topk_idx, int32_t *status, hipStream_t st) {
  hipLaunchKernelGGL(topk_check_kernel, dim3(1), dim3(1024), 0, st, topk_idx, s.T, s.H, s.expert_choice ? s.E : s.k,
                     s.Eh, s.expert_choice ? 1 : 0, status);
  return launch_status("routing check");
}

// ---------------------------------------------------------------- host
static long n_chunks(const Shape &s) { return ((long)s.T * s.K + CH - 1) / CH; }

size_t dispatch_ws_bytes(const Shape &s) {
  size_t b = align_up((size_t)n_chunks(s) * s.E * 4, 256);  // chunk histograms
  b += align_up((size_t)(s.E + 1) * 4, 256);                  // all_off
  if (s.drop >= DROP_AFFINITY) b += align_up((size_t)s.T * s.K * 4, 256);  // expert-sorted segments
  return b;
}

template <typename TA>
static void launch_scatter(const Shape &s, const void *x, const int32_t *row_of, void *x_perm, hipStream_t st) {
  const long total = (long)s.T * (s.H * s.dh * (long)sizeof(TA) / 16);
  long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
#define SC(KH_)                                                                                              \
  hipLaunchKernelGGL((disp_scatter_kernel<TA, KH_>), dim3(blocks), dim3(256), 0, st, (const TA *)x, row_of, \
                     (TA *)x_perm, s.T, s.H, s.k, s.dh, s.R_max)
  if (s.k <= 1) SC(1);
  else if (s.k <= 2) SC(2);
  else if (s.k <= 4) SC(4);
  else if (s.k <= 8) SC(8);
  else SC(0);
#undef SC
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
  int32_t *seg = (s.drop >= DROP_AFFINITY) ? (int32_t *)p : nullptr;

  if (s.expert_choice) {
    // the slots are fixed (slot j of every token is expert j): counts in closed form, no ranking
    hipLaunchKernelGGL(disp_ec_counts_kernel, dim3(1), dim3(256), 0, st, s.E, s.T, s.C, demand, counts, offsets,
                       all_off);
    if (int rc = launch_status("dispatch counts")) return rc;
  } else {
    hipLaunchKernelGGL(disp_hist_kernel, dim3(nc), dim3(256), s.E * 4, st, topk_idx, n, s.E, hist);
    if (int rc = launch_status("dispatch histogram")) return rc;
    hipLaunchKernelGGL(disp_rank_kernel, dim3(nc), dim3(256), 9 * s.E * 4, st, topk_idx, n, s.E, (int)nc, hist,
                       s.drop, s.C, s.keep_num, s.keep_den, demand, counts, offsets, all_off, row_of, src_of, seg);
    if (int rc = launch_status("dispatch rank")) return rc;
  }
  if (s.drop >= DROP_AFFINITY) {
    // an expert holds at most T assignments (one per token of its head)
    const int cap = (int)std::min<long>(std::max(s.T, 1), AFF_LDS_MAX);
    // experts holding thousands of assignments each (expert choice: T) take 1024-thread blocks
    const int ecE = s.expert_choice ? s.E : 0;
    if (s.drop == DROP_TOPC || n / s.E >= 4096)
      hipLaunchKernelGGL(disp_affinity_kernel<1024>, dim3(s.E), dim3(1024), (size_t)cap * 8, st, seg, all_off,
                         counts, offsets, topk_w, row_of, src_of, cap, ecE);
    else
      hipLaunchKernelGGL(disp_affinity_kernel<256>, dim3(s.E), dim3(256), (size_t)cap * 8, st, seg, all_off,
                         counts, offsets, topk_w, row_of, src_of, cap, ecE);
    if (int rc = launch_status("dispatch affinity")) return rc;
  }
  if (x_perm) {
    if (s.act_f32) launch_scatter<float>(s, x, row_of, x_perm, st);
    else launch_scatter<uint16_t>(s, x, row_of, x_perm, st);
    if (int rc = launch_status("dispatch scatter")) return rc;
  }
  return 0;
}

}  // namespace moe

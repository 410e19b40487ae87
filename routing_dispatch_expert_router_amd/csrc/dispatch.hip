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
// Pipeline (flat assignment a = t*K + j):
//   hist      per-chunk expert histogram of HIST_CA consecutive a (LDS integer
//             atomics: order-free); skipped when the router's per-block choice
//             counts are at hand (the layer), which are the same histogram
//             over chunks of its blocks' tokens
//   rank      each block adds the histograms of the chunks before its own (its
//             base per expert) and of all chunks (the demand), applies the keep
//             rule to the demand and scans the kept counts into offsets (block
//             0 writes demand, counts, offsets); then the stable rank of every
//             a among the earlier a of its expert = base + per-wave prefix +
//             in-wave ballot match; writes row_of / src_of (NONE, CAPACITY) or
//             the expert-sorted segment list (AFFINITY)
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

// ---------------------------------------------------------------- counting and ranking
// A chunk histogram hist[q][E] holds the expert counts of the assignments
// [q*ca, (q+1)*ca).  disp_hist_kernel writes one with ca = HIST_CA; the
// router writes one as a by-product (each of its blocks counts the choices
// of its tokens: ca = tokens per router block x K), which lets the layer skip
// the histogram launch.
constexpr int HIST_CA = 1024;     // assignments per histogram block (256 threads x 4)
constexpr int RANK_NT = 256;      // threads per ranking block
constexpr int RANK_WAVES = RANK_NT / 64;
constexpr int RANK_TARGET = 1024; // assignments per ranking block, about
constexpr int RANK_PF = 4;        // expert ids per lane held in registers (256 per wave)

__global__ __launch_bounds__(256) void disp_hist_kernel(const int32_t *__restrict__ idx, long n, int E,
                                                        int32_t *__restrict__ hist) {
  extern __shared__ int32_t h[];
  const long a0 = (long)blockIdx.x * HIST_CA + threadIdx.x;
  int ev[HIST_CA / 256];
#pragma unroll
  for (int i = 0; i < HIST_CA / 256; ++i) ev[i] = a0 + i * 256 < n ? idx[a0 + i * 256] : -1;
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < HIST_CA / 256; ++i)
    if (ev[i] >= 0) atomicAdd(&h[ev[i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(long)blockIdx.x * E + e] = h[e];
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

// Exclusive scans of two values per thread over a RANK_NT-thread block (thread
// order) and their totals; integer sums, so the order of the additions does
// not matter.  wsum is not reused afterwards.
__device__ __forceinline__ int2 rank_block_scan2(int v0, int v1, int2 *wsum, int2 *total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x0 = v0, x1 = v1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y0 = __shfl_up(x0, o), y1 = __shfl_up(x1, o);
    if (lane >= o) {
      x0 += y0;
      x1 += y1;
    }
  }
  if (lane == 63) wsum[w] = make_int2(x0, x1);
  __syncthreads();
  int b0 = 0, b1 = 0, t0 = 0, t1 = 0;
#pragma unroll
  for (int q = 0; q < RANK_WAVES; ++q) {
    const int2 s = wsum[q];
    b0 += q < w ? s.x : 0;
    b1 += q < w ? s.y : 0;
    t0 += s.x;
    t1 += s.y;
  }
  *total = make_int2(t0, t1);
  return make_int2(b0 + x0 - v0, b1 + x1 - v1);
}

// Geometry of the histogram read: groups of W consecutive experts (W = 4
// when E is a multiple of 4: 16-byte loads), P parts per group; thread
// (part p, group g) adds chunks p, p + P, ...
struct RankGeom {
  int W, G, P;
};
__host__ __device__ inline RankGeom rank_geom(int E, int nq) {
  RankGeom r;
  r.W = (E % 4 == 0) ? 4 : 1;
  r.G = E / r.W;
  r.P = RANK_NT / r.G > 0 ? RANK_NT / r.G : 1;
  if (r.P > nq) r.P = nq > 0 ? nq : 1;
  return r;
}
// dynamic LDS of disp_rank_kernel, in ints: per-wave counts [4][E], the two
// partial-sum matrices [P][E], offsets [2][E]
__host__ __device__ inline long rank_lds_ints(int E, int nq) {
  return (long)RANK_WAVES * E + 2L * rank_geom(E, nq).P * E + 2L * E;
}

// One block (4 waves) per m consecutive histogram chunks; wave w owns the
// w-th quarter of the block's assignments.  The block adds the chunk
// histograms (the earlier chunks: its base per expert; all: the demand),
// applies the keep rule and scans the kept counts into offsets (block 0
// writes demand, counts, offsets); each wave counts its own assignments per
// expert, and the stable rank of an assignment among the earlier ones of its
// expert is base + the earlier waves' counts + the earlier steps of its wave
// + the lower lanes of its step holding the same expert (ballot match).
// Writes row_of / src_of (NONE, CAPACITY) or the expert-sorted segment list
// (AFFINITY).
__global__ __launch_bounds__(RANK_NT) void disp_rank_kernel(
    const int32_t *__restrict__ idx, long n, int E, const int32_t *__restrict__ hist, int nq, long ca, int m,
    int drop, int C, int keep_num, int keep_den, int32_t *__restrict__ demand, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ all_off_out, int32_t *__restrict__ row_of,
    int32_t *__restrict__ src_of, int32_t *__restrict__ seg) {
  extern __shared__ int32_t sm[];
  const RankGeom rg = rank_geom(E, nq);
  int32_t *cnt = sm;                         // [4][E] per-wave counts, then running ranks
  int32_t *pb = cnt + RANK_WAVES * E;        // [P][E] partial sums over the earlier chunks
  int32_t *pt = pb + (size_t)rg.P * E;       // [P][E] partial sums over all chunks
  int32_t *off = pt + (size_t)rg.P * E;      // [E] first row of each expert
  int32_t *aoff = off + E;                   // [E] first slot of each expert in the affinity segments
  __shared__ int2 wsum[RANK_WAVES];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q0 = blockIdx.x * m;
  const long a_beg = (long)q0 * ca, a_end = min(n, (long)min(nq, q0 + m) * ca);
  const long sg = (a_end - a_beg + RANK_WAVES - 1) / RANK_WAVES;
  const long s0 = min(a_end, a_beg + (long)w * sg), s1 = min(a_end, s0 + sg);
  // the wave's first RANK_PF * 64 expert ids, loaded once
  int ev[RANK_PF];
#pragma unroll
  for (int i = 0; i < RANK_PF; ++i) {
    const long a = s0 + i * 64 + lane;
    ev[i] = a < s1 ? idx[a] : 0;
  }
  // partial sums of the chunk histograms (coalesced rows, W experts per load):
  // slot (part p, group g) adds chunks p, p + P, ...; P * G <= max(RANK_NT, G)
  for (int slot = tid; slot < rg.P * rg.G; slot += RANK_NT) {
    int sb[4] = {0, 0, 0, 0}, st[4] = {0, 0, 0, 0};
    const int g = slot % rg.G, p = slot / rg.G;
    if (rg.W == 4) {
#pragma unroll 16
      for (int q = p; q < nq; q += rg.P) {
        const int4 v = reinterpret_cast<const int4 *>(hist + (size_t)q * E)[g];
        const bool before = q < q0;
        st[0] += v.x; st[1] += v.y; st[2] += v.z; st[3] += v.w;
        sb[0] += before ? v.x : 0; sb[1] += before ? v.y : 0;
        sb[2] += before ? v.z : 0; sb[3] += before ? v.w : 0;
      }
    } else {
#pragma unroll 16
      for (int q = p; q < nq; q += rg.P) {
        const int v = hist[(size_t)q * E + g];
        st[0] += v;
        sb[0] += q < q0 ? v : 0;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < rg.W) {
        pb[(size_t)p * E + g * rg.W + j] = sb[j];
        pt[(size_t)p * E + g * rg.W + j] = st[j];
      }
  }
  // per-wave counts of the wave's own assignments (the row is the wave's own)
  for (int e = lane; e < E; e += 64) cnt[w * E + e] = 0;
#pragma unroll
  for (int i = 0; i < RANK_PF; ++i)
    if (s0 + i * 64 + lane < s1) atomicAdd(&cnt[w * E + ev[i]], 1);
  for (long a = s0 + RANK_PF * 64 + lane; a < s1; a += 64) atomicAdd(&cnt[w * E + idx[a]], 1);
  __syncthreads();
  // base (earlier chunks) and demand of every expert: groups of L lanes (L the
  // power of two >= P, at most 64) add the P partial sums of one expert each
  {
    int L = 1;
    while (L < rg.P && L < 64) L <<= 1;
    const int per = 64 / L, sub = lane % L;
    for (int e0 = w * per; e0 < E; e0 += RANK_WAVES * per) {  // wave-uniform
      const int e = e0 + lane / L;
      int vb = 0, vt = 0;
      if (e < E)
        for (int p = sub; p < rg.P; p += L) {
          vb += pb[(size_t)p * E + e];
          vt += pt[(size_t)p * E + e];
        }
      for (int o = L >> 1; o > 0; o >>= 1) {
        vb += __shfl_xor(vb, o);
        vt += __shfl_xor(vt, o);
      }
      if (e < E && sub == 0) {
        off[e] = vb;   // base, until the offsets replace it
        aoff[e] = vt;  // demand, until the segment offsets replace it
      }
    }
  }
  __syncthreads();
  // experts 4*tid .. 4*tid + 3: kept counts, and the per-wave counts turned
  // into running ranks
  int kept[4], tot[4];
  int skept = 0, stot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    kept[i] = tot[i] = 0;
    if (e < E) {
      const int vt = aoff[e];
      tot[i] = vt;
      kept[i] = drop == DROP_NONE       ? vt
                : drop == DROP_AFFINITY ? (int)(((long)keep_num * vt + keep_den - 1) / keep_den)
                                        : min(vt, C);  // capacity
      int run = off[e];
#pragma unroll
      for (int q = 0; q < RANK_WAVES; ++q) {
        const int v = cnt[q * E + e];
        cnt[q * E + e] = run;
        run += v;
      }
    }
    skept += kept[i];
    stot += tot[i];
  }
  int2 total;
  const int2 ex = rank_block_scan2(skept, stot, wsum, &total);
  {
    int ok = ex.x, ot = ex.y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < E) {
        off[e] = ok;
        aoff[e] = ot;
        if (blockIdx.x == 0) {
          demand[e] = tot[i];
          counts[e] = kept[i];
          offsets[e] = ok;
          if (drop >= DROP_AFFINITY) all_off_out[e] = ot;
        }
      }
      ok += kept[i];
      ot += tot[i];
    }
  }
  if (blockIdx.x == 0 && tid == 0) {
    offsets[E] = total.x;
    if (drop >= DROP_AFFINITY) all_off_out[E] = (int)n;
  }
  __syncthreads();
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  auto rank_step = [&](long a, int e, bool act) {
    const uint64_t mm = match_mask(e, act);
    const int before = __popcll(mm & lt);
    int rank = 0;
    if (act) rank = cnt[w * E + e] + before;
    // the highest lane of each group advances the counter (after every lane read it)
    const bool leader = act && ((mm >> lane) >> 1) == 0ull;
    if (leader) cnt[w * E + e] = rank + 1;
    if (act) {
      if (drop >= DROP_AFFINITY) {
        seg[aoff[e] + rank] = (int32_t)a;
      } else {
        const bool kp = (drop == DROP_NONE) || rank < C;
        const int row = kp ? off[e] + rank : -1;
        row_of[a] = row;
        if (kp) src_of[row] = (int32_t)a;
      }
    }
  };
#pragma unroll
  for (int i = 0; i < RANK_PF; ++i) {
    if (s0 + i * 64 >= s1) break;  // wave-uniform
    const long a = s0 + i * 64 + lane;
    rank_step(a, ev[i], a < s1);
  }
  for (long a0 = s0 + RANK_PF * 64; a0 < s1; a0 += 64) {  // wave-uniform
    const long a = a0 + lane;
    const bool act = a < s1;
    rank_step(a, act ? idx[a] : 0, act);
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
static long n_chunks(const Shape &s) { return ((long)s.T * s.K + HIST_CA - 1) / HIST_CA; }

static size_t dispatch_tail_bytes(const Shape &s) {
  size_t b = align_up((size_t)(s.E + 1) * 4, 256);                         // all_off
  if (s.drop >= DROP_AFFINITY) b += align_up((size_t)s.T * s.K * 4, 256);  // expert-sorted segments
  return b;
}

size_t dispatch_ws_bytes(const Shape &s) {
  return align_up((size_t)n_chunks(s) * s.E * 4, 256) + dispatch_tail_bytes(s);  // + chunk histograms
}

size_t dispatch_after_route_ws_bytes(const Shape &s) { return route_stats_bytes(s) + dispatch_tail_bytes(s); }

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
                    void *x_perm, void *ws, hipStream_t st, const int32_t *route_hist) {
  const long n = (long)s.T * s.K;
  const bool rh = route_hist != nullptr;
  const RouteGeom rgeo = route_geometry(s);
  // chunk histograms: the router's (chunks of its blocks' tokens) or this call's own
  const long nq = rh ? rgeo.nbx : n_chunks(s);
  const long ca = rh ? (long)rgeo.tb * s.K : HIST_CA;
  char *p = (char *)ws;
  const int32_t *hist = rh ? route_hist : (const int32_t *)p;
  p += rh ? route_stats_bytes(s) : align_up((size_t)nq * s.E * 4, 256);
  int32_t *all_off = (int32_t *)p;
  p += align_up((size_t)(s.E + 1) * 4, 256);
  int32_t *seg = (s.drop >= DROP_AFFINITY) ? (int32_t *)p : nullptr;

  if (s.expert_choice) {
    // the slots are fixed (slot j of every token is expert j): counts in closed form, no ranking
    hipLaunchKernelGGL(disp_ec_counts_kernel, dim3(1), dim3(256), 0, st, s.E, s.T, s.C, demand, counts, offsets,
                       all_off);
    if (int rc = launch_status("dispatch counts")) return rc;
  } else {
    if (!rh) {
      hipLaunchKernelGGL(disp_hist_kernel, dim3((unsigned)nq), dim3(256), s.E * 4, st, topk_idx, n, s.E,
                         const_cast<int32_t *>(hist));
      if (int rc = launch_status("dispatch histogram")) return rc;
    }
    const int m = (int)std::max<long>(1, RANK_TARGET / ca);
    const long nb = (nq + m - 1) / m;
    const size_t lds = (size_t)rank_lds_ints(s.E, (int)nq) * 4;
    hipLaunchKernelGGL(disp_rank_kernel, dim3((unsigned)nb), dim3(RANK_NT), lds, st, topk_idx, n, s.E, hist,
                       (int)nq, ca, m, s.drop, s.C, s.keep_num, s.keep_den, demand, counts, offsets, all_off, row_of,
                       src_of, seg);
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

// Beam-search survivor selection with early termination (xGR page, section
// 2.2 xBeam: Top-K selection from the pool of every live beam's candidates;
// a beam's candidates arrive sorted, so its walk stops at the first one that
// cannot enter the current best set, and most of the pool is never sorted).
//
// One workgroup per request. Keys are 64-bit: the candidate score in an
// order-preserving unsigned form on top, the complement of its pool index
// below, so every key is distinct and "larger key" means "higher score, then
// smaller index" - exactly the required order.
//  1. Seed: the best few candidates of every beam (about 4 * n_out keys). If
//     there are at least n_out of them, the n_out-th largest is a lower bound
//     tau for the n_out-th largest key of the whole pool.
//  2. Walk: beams are scanned in rounds of kChunk candidates; a beam takes
//     part in the next round only while its last scanned candidate still
//     reaches tau (early termination). Candidates with key >= tau are
//     appended to LDS.
//  3. Sort the survivors (bitonic, in LDS) and emit the n_out largest.
// If the survivors do not fit in LDS (many exact ties), a slower exact path
// merges blocks of beams into a running best set instead.
#include "device.h"
#include "kernels.h"

namespace xattn {

namespace {

constexpr int kThreads = 1024;
constexpr int kChunk = 16;  // candidates per beam per walk round

__device__ __forceinline__ uint32_t ordered_bits(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;  // -0.0 and +0.0 are the same score
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float s, uint32_t idx) {
  return ((uint64_t)ordered_bits(s) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Bitonic sort of keys[0, n) into descending order; n is a power of two,
// at most kTopkCap. Whole workgroup. Element i lives in thread i % kThreads
// (slot i / kThreads) while it is in registers, so every compare-exchange at
// a stride below 64 pairs two lanes of one wavefront and runs on register
// shuffles with no barrier; strides of 64 and more go through LDS.
constexpr int kSortSlots = kTopkCap / kThreads;

__device__ __forceinline__ void reg_steps(uint64_t* v, int n, int size, int smax) {
  const int tid = threadIdx.x;
  for (int stride = smax; stride >= 1; stride >>= 1) {
#pragma unroll
    for (int q = 0; q < kSortSlots; ++q) {
      if (q * kThreads < n) {  // uniform
        const int i = q * kThreads + tid;
        const uint64_t p = __shfl_xor(v[q], stride);
        const bool keep_max = ((i & size) == 0) == ((i & stride) == 0);
        v[q] = keep_max ? (v[q] > p ? v[q] : p) : (v[q] < p ? v[q] : p);
      }
    }
  }
}

__device__ __forceinline__ void load_regs(uint64_t* v, const uint64_t* keys, int n) {
#pragma unroll
  for (int q = 0; q < kSortSlots; ++q) {
    const int i = q * kThreads + threadIdx.x;
    v[q] = i < n ? keys[i] : 0ull;
  }
}

__device__ __forceinline__ void store_regs(const uint64_t* v, uint64_t* keys, int n) {
#pragma unroll
  for (int q = 0; q < kSortSlots; ++q) {
    const int i = q * kThreads + threadIdx.x;
    if (i < n) keys[i] = v[q];
  }
}

// Bitonic sort of 64 * S keys held by one wavefront, S per lane (element
// e = S * lane + s), into descending order: strides below S swap inside a
// lane, larger ones pair lanes through shuffles. No barrier and no LDS, which
// for a few hundred keys beats the workgroup sort's barrier-bound stages.
template <int S>
__device__ __forceinline__ void wave_sort_desc(uint64_t* v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64 * S; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride >= 1; stride >>= 1) {
      if (stride < S) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
          if (s & stride) continue;
          const int e = S * lane + s;
          const bool desc = (e & size) == 0;
          const uint64_t a = v[s], b = v[s + stride];
          const bool swap = desc ? a < b : a > b;
          v[s] = swap ? b : a;
          v[s + stride] = swap ? a : b;
        }
      } else {
        const int lm = stride / S;
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int e = S * lane + s;
          const uint64_t p = __shfl_xor(v[s], lm);
          const bool keep_max = ((e & size) == 0) == ((e & stride) == 0);
          v[s] = keep_max ? (v[s] > p ? v[s] : p) : (v[s] < p ? v[s] : p);
        }
      }
    }
  }
}

// The n (<= 64 * S) keys of keys_in[] (or computed by key_of(i)) sorted by
// wave 0; the first n_keep land in out[] in order. Other waves do nothing.
template <int S, typename F>
__device__ __forceinline__ void wave_sort_to(F&& key_of, int n, uint64_t* out, int n_keep) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  uint64_t v[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = S * lane + s;
    v[s] = e < n ? key_of(e) : 0ull;
  }
  wave_sort_desc<S>(v);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = S * lane + s;
    if (e < n_keep) out[e] = v[s];
  }
}

// Caller: keys[0, n) written and visible (a barrier since). Ends with a
// barrier, the sorted keys in LDS.
__device__ void sort_desc(uint64_t* keys, int n) {
  uint64_t v[kSortSlots];
  load_regs(v, keys, n);
  for (int size = 2; size <= n && size <= 64; size <<= 1) reg_steps(v, n, size, size >> 1);
  __syncthreads();  // every load done before any store
  store_regs(v, keys, n);
  __syncthreads();
  for (int size = 128; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride >= 64; stride >>= 1) {
      for (int t = threadIdx.x; t < (n >> 1); t += blockDim.x) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool desc = (i & size) == 0;
        const uint64_t a = keys[i], b = keys[j];
        if ((a < b) == desc) {
          keys[i] = b;
          keys[j] = a;
        }
      }
      __syncthreads();
    }
    load_regs(v, keys, n);
    reg_steps(v, n, size, 32);
    __syncthreads();
    store_regs(v, keys, n);
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void beam_topk_kernel(TopkArgs a) {
  __shared__ uint64_t keys[kTopkCap];
  __shared__ __attribute__((aligned(16))) int act[2][kTopkMaxBeams];  // beams still walking, per round parity
  __shared__ int s_count, s_nact[2];
  const int r = blockIdx.x;
  const int BW = a.BW, K = a.K, N = a.n_out;
  const int tid = threadIdx.x;
  const float* bs = a.beam_score + (int64_t)r * BW;
  const float* lp = a.logprob + (int64_t)r * BW * K;

  // 1. Seed threshold from a sample: the best m candidates of every beam
  //    (m chosen so the sample holds about 4 * n_out keys and fits in LDS).
  //    Its n_out-th largest key bounds the pool's from below.
  uint64_t tau = 0;
  int m = (4 * N + BW - 1) / BW;
  m = max(1, min(m, min(K, kTopkCap / BW)));
  const int n_s = BW * m;
  if (n_s >= N) {
    auto sample = [&](int i) {
      const int b = i / m, k = i - (i / m) * m;
      return make_key(bs[b] + lp[(int64_t)b * K + k], (uint32_t)b * (uint32_t)K + (uint32_t)k);
    };
    if (n_s <= 512) {
      wave_sort_to<8>(sample, n_s, keys, N);
    } else if (n_s <= 1024) {
      wave_sort_to<16>(sample, n_s, keys, N);
    } else {
      const int n2 = next_pow2(n_s);
      for (int i = tid; i < n2; i += kThreads) keys[i] = i < n_s ? sample(i) : 0ull;
      __syncthreads();
      sort_desc(keys, n2);
    }
    __syncthreads();
    tau = keys[N - 1];
    __syncthreads();
  }

  // 2. Walk with early termination. Round 0 scans the first kChunk
  //    candidates of every beam; each later round splits the workgroup's
  //    kThreads * 4 candidate slots evenly over the beams still going (a
  //    beam goes on while the last candidate it scanned reaches tau and
  //    candidates remain), so a few strong beams finish in few rounds.
  if (tid == 0) {
    s_count = 0;
    s_nact[0] = s_nact[1] = 0;
  }
  __syncthreads();
  bool overflow = false;
  int n_found = 0;
  int n_act = BW;  // beams in this round (round 0: all, in order)
  int pos = 0;     // first candidate of this round (the same for every beam)
  for (int round = 0;; ++round) {
    const int chunk = round == 0 ? kChunk : max(kChunk, ((kThreads * 4) / n_act) & ~3);
    const int Q = chunk / 4;
    for (int u = tid; u < n_act * Q; u += kThreads) {
      const int ai = u / Q, q = u - ai * Q;
      const int b = round == 0 ? ai : act[round & 1][ai];
      const float sb = bs[b];
      const int k0 = pos + 4 * q;
      uint64_t kk[4];
      int nk = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = k0 + e;
        kk[e] = 0;
        if (k < K) {
          kk[e] = make_key(sb + lp[(int64_t)b * K + k], (uint32_t)b * (uint32_t)K + (uint32_t)k);
          nk += kk[e] >= tau ? 1 : 0;
        }
      }
      if (nk > 0) {
        const int at = atomicAdd(&s_count, nk);
        int w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (k0 + e < K && kk[e] >= tau) {
            if (at + w < kTopkCap) keys[at + w] = kk[e];
            ++w;
          }
        }
      }
      if (q == Q - 1 && k0 + 3 < K - 1 && kk[3] >= tau)
        act[(round + 1) & 1][atomicAdd(&s_nact[(round + 1) & 1], 1)] = b;
    }
    __syncthreads();
    n_act = s_nact[(round + 1) & 1];
    n_found = s_count;
    if (tid == 0) s_nact[round & 1] = 0;  // the counter the next round appends to
    __syncthreads();
    pos += chunk;
    if (n_found > kTopkCap) {
      overflow = true;
      break;
    }
    if (n_act == 0) break;
  }

  int n_top;
  if (!overflow) {
    // 3. Sort the survivors; the n_out largest lead.
    const int n = n_found;
    if (n <= 1024) {
      // One wave sorts them in registers into the other buffer (act, free
      // after the walk).
      uint64_t* sorted = reinterpret_cast<uint64_t*>(&act[0][0]);
      auto survivor = [&](int i) { return keys[i]; };
      if (n <= 512)
        wave_sort_to<8>(survivor, n, sorted, N);
      else
        wave_sort_to<16>(survivor, n, sorted, N);
      __syncthreads();
      for (int i = tid; i < N; i += kThreads) keys[i] = sorted[i];
      __syncthreads();
    } else {
      const int n2 = next_pow2(n);
      for (int i = n + tid; i < n2; i += kThreads) keys[i] = 0ull;
      __syncthreads();
      sort_desc(keys, n2);
    }
    n_top = N;
  } else {
    // Exact fallback: merge blocks of whole beams into a running best set
    // held at keys[0, n_top). A block's candidates (at most kTopkCap - N of
    // them) always fit behind it.
    n_top = 0;
    const int per_block = (kTopkCap - N) / K;
    for (int b0 = 0; b0 < BW; b0 += per_block) {
      const int b1 = min(BW, b0 + per_block);
      __syncthreads();
      if (tid == 0) s_count = n_top;
      __syncthreads();
      for (int u = tid; u < (b1 - b0) * K; u += kThreads) {
        const int b = b0 + u / K, k = u - (u / K) * K;
        const uint64_t key = make_key(bs[b] + lp[(int64_t)b * K + k], (uint32_t)b * (uint32_t)K + (uint32_t)k);
        if (key >= tau) keys[atomicAdd(&s_count, 1)] = key;
      }
      __syncthreads();
      const int n = s_count;
      const int n2 = next_pow2(n);
      for (int i = n + tid; i < n2; i += kThreads) keys[i] = 0ull;
      __syncthreads();
      sort_desc(keys, n2);
      n_top = min(N, n);
      if (n_top == N && keys[N - 1] > tau) tau = keys[N - 1];
    }
  }

  // 4. Emit.
  for (int i = tid; i < n_top; i += kThreads) {
    const uint32_t idx = 0xFFFFFFFFu - (uint32_t)(keys[i] & 0xFFFFFFFFull);
    const int b = (int)(idx / (uint32_t)K), k = (int)(idx - (uint32_t)b * (uint32_t)K);
    const int64_t o = (int64_t)r * N + i;
    a.parent[o] = b;
    a.token_out[o] = a.token[((int64_t)r * BW + b) * K + k];
    a.score_out[o] = bs[b] + lp[(int64_t)b * K + k];
  }
}

}  // namespace

hipError_t launch_beam_topk(const TopkArgs& a, hipStream_t st) {
  if (a.R == 0 || a.n_out == 0) return hipSuccess;
  hipLaunchKernelGGL(beam_topk_kernel, dim3(a.R), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace xattn

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

// Sort keys[0, n) descending; n is a power of two. Whole workgroup.
__device__ void sort_desc(uint64_t* keys, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
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
  }
}

__global__ __launch_bounds__(kThreads) void beam_topk_kernel(TopkArgs a) {
  __shared__ uint64_t keys[kTopkCap];
  __shared__ uint8_t active[2][kTopkMaxBeams];
  __shared__ int s_count, s_more;
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
    const int n2 = next_pow2(n_s);
    for (int i = tid; i < n2; i += kThreads) {
      uint64_t key = 0ull;
      if (i < n_s) {
        const int b = i / m, k = i - (i / m) * m;
        key = make_key(bs[b] + lp[(int64_t)b * K + k], (uint32_t)b * (uint32_t)K + (uint32_t)k);
      }
      keys[i] = key;
    }
    __syncthreads();
    sort_desc(keys, n2);
    tau = keys[N - 1];
    __syncthreads();
  }

  // 2. Walk with early termination.
  if (tid == 0) s_count = 0;
  for (int b = tid; b < BW; b += kThreads) active[0][b] = 1;
  __syncthreads();
  bool overflow = false;
  int n_found = 0;
  constexpr int Q = kChunk / 4;  // quads of candidates per beam per round
  for (int j = 0, cur = 0; j * kChunk < K; ++j, cur ^= 1) {
    if (tid == 0) s_more = 0;
    for (int b = tid; b < BW; b += kThreads) active[cur ^ 1][b] = 0;
    __syncthreads();
    for (int u = tid; u < BW * Q; u += kThreads) {
      const int b = u / Q, q = u - b * Q;
      if (!active[cur][b]) continue;
      const float sb = bs[b];
      const int k0 = j * kChunk + 4 * q;
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
        const int pos = atomicAdd(&s_count, nk);
        int w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (k0 + e < K && kk[e] >= tau) {
            if (pos + w < kTopkCap) keys[pos + w] = kk[e];
            ++w;
          }
        }
      }
      // the beam goes on only if its last candidate of this round still
      // reaches tau and candidates remain
      if (q == Q - 1 && k0 + 3 < K - 1 && kk[3] >= tau) {
        active[cur ^ 1][b] = 1;
        s_more = 1;
      }
    }
    __syncthreads();
    const int more = s_more;
    n_found = s_count;
    __syncthreads();  // every thread has read both before thread 0 resets them
    if (n_found > kTopkCap) {
      overflow = true;
      break;
    }
    if (!more) break;
  }

  int n_top;
  if (!overflow) {
    // 3. Sort the survivors; the n_out largest lead.
    const int n = n_found;
    const int n2 = next_pow2(n);
    for (int i = n + tid; i < n2; i += kThreads) keys[i] = 0ull;
    __syncthreads();
    sort_desc(keys, n2);
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

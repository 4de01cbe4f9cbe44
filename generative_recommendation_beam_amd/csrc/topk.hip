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
//  3. Order the survivors and emit the n_out largest: for n_out <= 512,
//     waves sort runs of 128, 256 or 512 keys in registers and pairwise
//     merges keep the best run; otherwise one wave sorts up to 1024 in
//     registers, or the workgroup sorts in LDS.
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

// The value lane ^ lm holds (lm a power of two below 64), by ALU lane
// exchanges only: data-parallel row permutes for 1, 2, 4 and 8, the
// half-swapping lane permutes for 16 and 32.
__device__ __forceinline__ uint32_t xor_lanes32(uint32_t v, int lm) {
  const int x = (int)v;
  switch (lm) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    case 4:  // half-row mirror (lane ^ 7), then quad_perm [3,2,1,0] (lane ^ 3)
      return (uint32_t)__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false), 0x1B, 0xF,
                                                0xF, false);
    case 8: return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row rotate by 8
    case 16: {  // odd 16-lane rows of one copy swapped with even rows of the other
      const auto w = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (threadIdx.x & 16) ? w[0] : w[1];
    }
    default: {  // upper 32 lanes of one copy swapped with the lower 32 of the other
      const auto w = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (threadIdx.x & 32) ? w[0] : w[1];
    }
  }
}

// ALU: the ALU exchanges above where lm is a compile-time constant (the
// generated networks below); else one LDS permute (a run-time lm would
// branch per exchange).
template <bool ALU>
__device__ __forceinline__ uint64_t xor_lanes(uint64_t v, int lm) {
  if (ALU && __builtin_constant_p(lm))  // (a run-time lm would branch per exchange)
    return ((uint64_t)xor_lanes32((uint32_t)(v >> 32), lm) << 32) | xor_lanes32((uint32_t)v, lm);
  return __shfl_xor(v, lm);
}

// Bitonic sort of 64 * S keys held by one wavefront, S per lane (element
// e = S * lane + s), into descending order: strides below S swap inside a
// lane, larger ones pair lanes through lane exchanges. No barrier and no
// LDS. The whole wavefront must be active.
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

// The same network, generated at compile time (every lane distance a
// constant, so the ALU exchanges apply): stage STRIDE of the merge of
// descending runs of SIZE, or of one descending merge when SIZE = 0.
template <int S, bool ALU, int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_stage(uint64_t* v, int lane) {
  if constexpr (STRIDE < S) {  // inside a lane
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (s & STRIDE) continue;
      const int e = S * lane + s;
      const bool desc = SIZE == 0 || (e & SIZE) == 0;
      const uint64_t a = v[s], b = v[s + STRIDE];
      const bool swap = desc ? a < b : a > b;
      v[s] = swap ? b : a;
      v[s + STRIDE] = swap ? a : b;
    }
  } else {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int e = S * lane + s;
      const uint64_t p = xor_lanes<ALU>(v[s], STRIDE / S);
      const bool keep_max = (SIZE == 0 || (e & SIZE) == 0) == ((e & STRIDE) == 0);
      v[s] = keep_max ? (v[s] > p ? v[s] : p) : (v[s] < p ? v[s] : p);
    }
  }
}
template <int S, bool ALU, int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_stages(uint64_t* v, int lane) {  // STRIDE, STRIDE / 2, ..., 1
  bitonic_stage<S, ALU, SIZE, STRIDE>(v, lane);
  if constexpr (STRIDE > 1) bitonic_stages<S, ALU, SIZE, STRIDE / 2>(v, lane);
}
template <int S, bool ALU, int SIZE = 2>
__device__ __forceinline__ void bitonic_sort_desc(uint64_t* v, int lane) {
  bitonic_stages<S, ALU, SIZE, SIZE / 2>(v, lane);
  if constexpr (SIZE < 64 * S) bitonic_sort_desc<S, ALU, SIZE * 2>(v, lane);
}

// The n_keep (<= RL = 64 S) largest of n (<= 16 RL) keys (key i =
// key_of(i)) into out[0, n_keep), in descending order; runs[0, 16 RL) is LDS
// scratch (out may be runs itself, then n_keep = 0 and run 0 holds the
// result). Waves 0 .. nr-1 each sort a run of RL keys in registers, S per
// lane; then rounds of pairwise merges keep the RL largest of two runs: with
// A and B descending, max(A[i], B[RL-1-i]) is a bitonic sequence holding
// exactly the RL largest of both, which one bitonic merge puts in order.
// Whole workgroup (16 waves); ends with a barrier.
template <int S, typename F>
__device__ void topn_to(F&& key_of, int n, uint64_t* runs, uint64_t* out, int n_keep) {
  constexpr int RL = 64 * S;
  constexpr bool ALU = true;  // compile-time networks: ALU lane exchanges (measured faster for 2, 4 and 8 keys per lane)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int nr = (n + RL - 1) / RL;
  if (wave < nr) {  // uniform per wave
    uint64_t v[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int e = RL * wave + S * lane + s;
      v[s] = e < n ? key_of(e) : 0ull;
    }
    bitonic_sort_desc<S, ALU>(v, lane);
#pragma unroll
    for (int s = 0; s < S; ++s) runs[RL * wave + S * lane + s] = v[s];
  }
  __syncthreads();
  while (nr > 1) {
    const int nk = (nr + 1) >> 1;  // run k = best RL of runs 2k and 2k+1 (a missing one is all zeros)
    uint64_t v[S];
    if (wave < nk) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int i = S * lane + s;
        const uint64_t x = runs[2 * RL * wave + i];
        const uint64_t y = 2 * wave + 1 < nr ? runs[2 * RL * wave + 2 * RL - 1 - i] : 0ull;
        v[s] = x > y ? x : y;
      }
      bitonic_stages<S, ALU, 0, RL / 2>(v, lane);
    }
    __syncthreads();  // every read of this round before any write
    if (wave < nk) {
#pragma unroll
      for (int s = 0; s < S; ++s) runs[RL * wave + S * lane + s] = v[s];
    }
    __syncthreads();
    nr = nk;
  }
  for (int i = threadIdx.x; i < n_keep; i += blockDim.x) out[i] = runs[i];
  __syncthreads();
}

// topn_to with the smallest run that holds n_keep (<= 512) keys; false (and
// nothing done) when the n keys need more than 16 runs or n_keep > 512.
template <typename F>
__device__ bool topn_any(F&& key_of, int n, uint64_t* runs, uint64_t* out, int n_keep, int N) {
  if (N <= 128 && n <= 16 * 128) {
    topn_to<2>(key_of, n, runs, out, n_keep);
  } else if (N <= 256 && n <= 16 * 256) {
    topn_to<4>(key_of, n, runs, out, n_keep);
  } else if (N <= 512 && n <= 16 * 512) {
    topn_to<8>(key_of, n, runs, out, n_keep);
  } else {
    return false;
  }
  return true;
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

  // Round 0 of the walk (below) scans the first kChunk candidates of every
  // beam, thread t taking four of them; they do not depend on the seed, so
  // they are requested now (indices clamped; unused ones are ignored).
  constexpr int Q0 = kChunk / 4;
  float pre_sb, pre_l[4];
  {
    const int u = min(tid, BW * Q0 - 1);
    const int b = u / Q0, k0 = 4 * (u - b * Q0);
    pre_sb = bs[b];
#pragma unroll
    for (int e = 0; e < 4; ++e) pre_l[e] = lp[(int64_t)b * K + min(k0 + e, K - 1)];
  }

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
    if (topn_any(sample, n_s, keys, keys, 0, N)) {
      // run 0 (keys[0, N)) holds the sample's best, in order
    } else if (n_s <= 512) {
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
    const int nu = n_act * Q;
    const int lane = tid & 63;
    const uint64_t below = (1ull << lane) - 1;  // lanes below this one
    // Whole waves iterate together, so the appends go through one LDS atomic
    // per wave (a ballot-based prefix sum places each lane's keys).
    for (int u0 = 0; u0 < nu; u0 += kThreads) {
      const int u = u0 + tid;
      const bool on = u < nu;
      const int uc = on ? u : 0;
      const int ai = uc / Q, q = uc - ai * Q;
      const int b = round == 0 ? ai : min(max(act[round & 1][ai], 0), BW - 1);  // (clamped: loads stay in the pool)
      const int k0 = pos + 4 * q;
      float sb, l[4];
      if (round == 0 && u0 == 0) {  // uniform: the prefetched candidates
        sb = pre_sb;
#pragma unroll
        for (int e = 0; e < 4; ++e) l[e] = pre_l[e];
      } else {
        sb = bs[b];
#pragma unroll
        for (int e = 0; e < 4; ++e) l[e] = lp[(int64_t)b * K + min(k0 + e, K - 1)];
      }
      uint64_t kk[4];
      int nk = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = on && k0 + e < K;
        kk[e] = ok ? make_key(sb + l[e], (uint32_t)b * (uint32_t)K + (uint32_t)(k0 + e)) : 0ull;
        nk += ok && kk[e] >= tau ? 1 : 0;
      }
      const uint64_t m0 = __ballot(nk & 1), m1 = __ballot(nk & 2), m2 = __ballot(nk & 4);
      const int tot = __popcll(m0) + 2 * __popcll(m1) + 4 * __popcll(m2);
      if (tot > 0) {  // uniform per wave
        int base = 0;
        if (lane == 0) base = atomicAdd(&s_count, tot);
        int at = __builtin_amdgcn_readfirstlane(base) + __popcll(m0 & below) + 2 * __popcll(m1 & below) +
                 4 * __popcll(m2 & below);  // (every lane active here: lane 0's base)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (on && k0 + e < K && kk[e] >= tau) {
            if (at < kTopkCap) keys[at] = kk[e];
            ++at;
          }
        }
      }
      // The beam goes on if its last candidate here reaches tau and more remain.
      const bool go = on && q == Q - 1 && k0 + 3 < K - 1 && kk[3] >= tau;
      const uint64_t mg = __ballot(go);
      if (mg) {  // uniform per wave
        int base = 0;
        if (lane == 0) base = atomicAdd(&s_nact[(round + 1) & 1], (int)__popcll(mg));
        const int gb = __builtin_amdgcn_readfirstlane(base);  // lane 0's: read with every lane active
        if (go) act[(round + 1) & 1][gb + __popcll(mg & below)] = b;
      }
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
    auto survivor = [&](int i) { return keys[i]; };
    if (topn_any(survivor, n, reinterpret_cast<uint64_t*>(&act[0][0]), keys, N, N)) {
      // keys[0, N): the survivors' best, in order (runs in act, free after the walk)
    } else if (n <= 1024) {
      // One wave sorts them in registers into the other buffer (act, free
      // after the walk).
      uint64_t* sorted = reinterpret_cast<uint64_t*>(&act[0][0]);
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

// Shared stage on bf16 MFMA (xGR page, section 2.1 xAttention: the Shared
// cache holds the prompt once for all beams; the Shared stage computes local
// scores and max/sum statistics; matmul and softmax are fused). Because every
// beam of a request reads the same prompt KV, the B*G query rows of one
// (request, kv head) form a dense Q.K^T / P.V contraction: this kernel streams
// each prompt K/V tile from HBM into LDS once and lets all of the workgroup's
// query rows use it on the matrix cores.
//
// Work unit (one workgroup): (request r, kv head h, tile of 32*NW query rows,
// prompt split). Each wavefront owns 32 query rows and works in transposed
// form, S^T = K . Q^T and O^T += V^T . P^T, with v_mfma_f32_32x32x16_bf16:
//  - B operand of S^T: lane (hh = lane/32, c = lane%32) holds query row c,
//    head-dim elements [16*dc + 8*hh, +8) - loaded once, kept in registers;
//  - S^T accumulator: lane holds 16 keys of query column c, so the row max and
//    sum are lane-local except one exchange between the two lane halves;
//  - P^T (bf16) feeds the next MFMA straight from those registers; the V^T
//    operand is read from row-major V in LDS with ds_read_b64_tr_b16.
// K/V tiles (64 keys) move HBM -> LDS with buffer_load_dwordx4 ... lds (no
// register staging), double-buffered so tile i+1 is in flight while tile i is
// computed. With one key group, D = 128 and two stages, the walk over full
// tiles is software-pipelined by 32-key halves (one half's S^T MFMAs beside
// the previous half's softmax, its P.V beside the next half's row maximum),
// and a stage's refill is split: the K rows of tile i+2 are issued as soon
// as the first half of tile i has read its K, the V rows after the second
// half; each refill is awaited with its own load count.
//
// Online softmax with the exact running maximum as the exponent offset: the
// output is rescaled whenever a half tile raises a row's maximum (the branch
// is skipped when no row of the wave moves). The probabilities are rounded
// to bf16 for the P.V MFMAs, so the offset is kept exact rather than lazy:
// with an offset up to 8 (log2) below the maximum, the dominant key's weight
// 2^x is rounded too, and rows where one key carries most of the weight (V
// entries of up to ~30 in the outlier workloads) lost up to ~3e-2 absolute;
// with the exact maximum that key's weight is exactly 1.
//
// Non-Shared part (prompt split 0, or a member of its own, when fused): the
// beam's own generated tokens, gathered through its slot-table row, join the
// same softmax state after the prompt tiles - per wave on the vector ALU, or,
// with four key groups, four query heads per kv head and at most three
// tokens, as one masked 32-key block on the matrix cores.
//
// Prompt splits: with p_splits > 1 and mode FIXUP, every split writes its
// partial (normalized O, lse) to the workspace, and the last workgroup of a
// (request, kv head, row tile) to arrive - found with a wrapping atomic
// counter that returns to zero - merges all partials with the log-sum-exp
// rule and writes the final output. In mode PARTIAL each split only writes its
// partial slot for a later reduction.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace xattn {

namespace {

constexpr int BN = 64;  // keys per tile

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// LDS tile layout: row-major [key][d] (D*2 bytes per key, no padding), with
// the 16-byte chunks of each row permuted by an XOR of a few key bits:
// chunk c of key k sits at position c ^ swz(k). One direct load instruction
// fills 1 KiB = D*2-byte rows of 1024/(2D) keys in lane order, so each lane
// fetches the global chunk that belongs at its position; a group of lanes
// reads whole rows, fully coalesced. The swizzles make the MFMA operand reads
// conflict-free and keep every operand address a per-lane base XOR-ed with a
// compile-time constant plus an immediate offset.
//  K rows (A operand of S^T = K.Q^T, lanes = keys):  swz_k(k) = k & 15  (D=128)
//                                                      (k >> 1) & 7  (D=64)
//  V rows (source of the transposed reads):            swz_v(k) = 4 * (k & 3)  (D=128)
//                                                      4 * (k & 1)  (D=64)
template <int D>
struct TileGeom {
  static constexpr int NCH = D / 8;              // 16-byte chunks per K/V row
  static constexpr int ROWB = D * 2;             // bytes per row
  static constexpr int TILEB = BN * ROWB;        // bytes per K (or V) tile
  static constexpr int KPI = 1024 / ROWB;        // keys per direct load instruction
  static constexpr int NINST = TILEB / 1024;     // direct loads per tile per tensor
  static constexpr int BUFB = 2 * TILEB;         // K + V tile
};

template <int D>
__device__ __forceinline__ int swz_k(int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int key) { return D == 128 ? ((key & 3) << 2) : ((key & 1) << 2); }

// Per-lane LDS byte bases of the MFMA operands (see the kernel).
template <int D>
__device__ __forceinline__ int k_operand_base(int lane) {
  using TG = TileGeom<D>;
  const int ql = lane & 31, hh = lane >> 5;
  const int f = swz_k<D>(ql);
  return ql * TG::ROWB + 16 * (hh ^ (f & 1)) + 32 * (f >> 1);
}
template <int D>
__device__ __forceinline__ int v_operand_base(int lane) {
  using TG = TileGeom<D>;
  const int hh = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
  const int key0 = 4 * hh + (i16 >> 2);
  const int x = 2 * (g16 & 1) + ((i16 & 3) >> 1);
  return TG::TILEB + key0 * TG::ROWB + 16 * (x ^ swz_v<D>(key0)) + (i16 & 1) * 8;
}

// The lane index, computed afresh where keeping the kernel's copy (and what
// derives from it) alive would cost registers.
__device__ __forceinline__ int fresh_lane() {
  int l;
  __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// A workgroup loads KG consecutive 64-key tiles per step (a super-tile); its
// NW waves share the KG*NINST direct-load instructions per tensor. Wave w
// issues instructions i = w + NW*j; instruction i fills 1 KiB of tile
// sub = i / NINST at LDS offset (i % NINST) * 1024. Per-lane byte offsets of
// the global chunks (relative to the super-tile start) for each j, K then V,
// are loop-invariant.
template <int D, int NW, int KG>
struct LoadPlan {
  using TG = TileGeom<D>;
  static_assert(TG::NINST % NW == 0, "waves must divide the load instructions of a tile");
  static constexpr int NJ = KG * TG::NINST / NW;
  // tile index and the wave-independent part of the LDS offset of load j
  static constexpr int sub(int j) { return NW * j / TG::NINST; }
  static constexpr int lds_off(int j) { return sub(j) * TG::BUFB + (NW * j - sub(j) * TG::NINST) * 1024; }
  uint32_t k[NJ];
  uint32_t v[NJ];
  __device__ __forceinline__ void init(int wave, int lane) {
    const int kin = lane / TG::NCH;
    const int pos = lane % TG::NCH;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int key = (wave + NW * j - sub(j) * TG::NINST) * TG::KPI + kin;  // key within its tile
      const uint32_t t0 = (uint32_t)(sub(j) * TG::TILEB);  // global byte offset of that tile
      k[j] = t0 + (uint32_t)(key * TG::ROWB + (pos ^ swz_k<D>(key)) * 16);
      v[j] = t0 + (uint32_t)(key * TG::ROWB + (pos ^ swz_v<D>(key)) * 16);
    }
  }
};

typedef __attribute__((address_space(3))) char lds_char;

// vmcnt(n) as an s_waitcnt immediate (vmcnt in bits 3:0 and 15:14; expcnt
// in 6:4 and lgkmcnt in 11:8 left at their maxima, i.e. not waited for).
constexpr int vm_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

// Wait until at most N vector-memory operations are in flight. Through the
// builtin rather than inline assembly, so that the compiler's own wait
// insertion sees it: the loads it issued earlier (query rows, per-request
// values) then count as landed there, and it adds no waits of its own for
// them behind the direct-to-LDS loads that follow (which it does not track).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vm_imm(N));
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ void wait_vmem() { wait_vm<0>(); }

// Split partials that one workgroup hands to another are written and read
// with agent-coherent buffer accesses (cache policy sc1, what agent-scope
// atomic loads/stores use). The hand-over itself follows the agent-scope
// release/acquire pattern: writers wait for their stores, fence (release,
// agent) and arrive on a counter with an acquire-release atomic; the last
// arrival fences (acquire, agent) before it reads the partials back.
constexpr int kCoherent = 16;  // sc1
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const float* base, int64_t floats) {
  const int64_t bytes = floats * 4;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0,
                                           (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff), 0x00020000);
}

// The value of lane i ^ 32, through the gfx950 lane swap (register to
// register: an LDS permute would make the next wait on LDS reads also wait
// for it). The whole wavefront must be active.
__device__ __forceinline__ float xor32(float x) {
  const auto w = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, (__lane_id() & 32) ? w[0] : w[1]);
}

// Maximum / sum of a value over the two lane halves (lanes c and c + 32), in
// every lane: the lane swap of two copies leaves [lo | lo] in one and
// [hi | hi] in the other, so one max or add combines them (no select). The
// two results are copied out of the swap's vector into scalars before the
// bit casts: a bit cast applied to an element of that vector directly was
// measured to read element 0 for both.
__device__ __forceinline__ float max_halves(float x) {
  const unsigned a = __builtin_bit_cast(unsigned, x);
  const auto w = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  const unsigned w0 = w[0];
  const unsigned w1 = w[1];
  return fmaxf(__builtin_bit_cast(float, w0), __builtin_bit_cast(float, w1));
}
__device__ __forceinline__ float sum_halves(float x) {
  const unsigned a = __builtin_bit_cast(unsigned, x);
  const auto w = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  const unsigned w0 = w[0];
  const unsigned w1 = w[1];
  return __builtin_bit_cast(float, w0) + __builtin_bit_cast(float, w1);
}

// Online-softmax update for one 32-key half of a tile (S^T block `sb`, the
// 16 scores this lane holds for its query column): the offset moves (and the
// output so far is rescaled) when a score passes it, and the half's
// probabilities are packed to bf16 in pf for its P.V MFMAs.
template <int D, bool MASK>
__device__ __forceinline__ void half_softmax(f32x16_t& sb, int kb, f32x16_t* oacc, float& m_run, float& l_part,
                                             float c, int hh, int nvalid, bf16x8_t* pf) {
  constexpr int NDB = D / 32;
  if (MASK) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
      if (key >= nvalid) sb[i] = neg_inf();
    }
  }
  float mx = fmaxf(fmaxf(sb[0], sb[1]), sb[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, sb[i]), sb[i + 1]);
  mx = fmaxf(mx, sb[15]);
  mx = max_halves(mx) * c;
  if (__any(mx > m_run)) {
    const float mn = fmaxf(m_run, mx);
    const float alpha = exp2_approx(m_run - mn);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    l_part *= alpha;
    m_run = mn;
  }
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float p = exp2_approx(__builtin_fmaf(sb[i], c, -m_run));
    lsum += p;
    pf[i >> 3][i & 7] = (__bf16)p;
  }
  l_part += lsum;
}

// half_softmax followed by that half's P.V MFMAs. Processing the halves
// separately lets the vector-ALU softmax of one half overlap the matrix-core
// work of the other.
template <int D, bool MASK, bool NO_HI1 = false>
__device__ __forceinline__ void half_softmax_pv(const char* buf, int vbase, f32x16_t& sb, int kb,
                                                f32x16_t* oacc, float& m_run, float& l_part, float c,
                                                int hh, int nvalid) {
  using TG = TileGeom<D>;
  constexpr int NDB = D / 32;
  bf16x8_t pf[2];
  half_softmax<D, MASK>(sb, kb, oacc, m_run, l_part, c, hh, nvalid, pf);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const int vo = (vbase ^ (64 * db)) + (16 * (2 * kb + ch)) * TG::ROWB;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(buf + vo));
      // NO_HI1: keys 24..31 of the half are not there (their V operand is zero)
      const i16x4_t hi = (NO_HI1 && ch == 1)
                             ? i16x4_t{0, 0, 0, 0}
                             : __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(buf + vo + 8 * TG::ROWB));
      const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[ch], oacc[db], 0, 0, 0);
    }
}

// Does nothing: the hook of a step that starts no loads.
struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// One 64-key tile for one wavefront (32 query rows): S^T = K.Q^T on MFMA for
// both 32-key halves, then per half the online softmax and O^T += V^T.P^T.
// MASK: the tile holds only `nvalid` keys (the last tile of a range).
// after_s() runs once the S^T MFMAs are issued (the loop starts the next
// tile's V loads there).
template <int D, bool MASK, typename F = NoHook>
__device__ __forceinline__ void tile_step(const char* buf, int kbase, int vbase, const bf16x8_t* qf,
                                          f32x16_t* oacc, float& m_run, float& l_part, float c,
                                          int hh, int nvalid, F&& after_s = F()) {
  using TG = TileGeom<D>;
  constexpr int NDC = D / 16;
  f32x16_t sacc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
  }
  // All K operand reads go out before the first MFMA, so LDS latency is paid
  // once per tile rather than once per MFMA.
  bf16x8_t ka[NDC][2];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      ka[dc][kb] = *reinterpret_cast<const bf16x8_t*>(buf + (kbase ^ (32 * dc)) + kb * 32 * TG::ROWB);
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * NDC, 0);  // the LDS reads first
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc][kb], qf[dc], sacc[kb], 0, 0, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * NDC, 0);  // then the MFMAs
  after_s();
  half_softmax_pv<D, MASK>(buf, vbase, sacc[0], 0, oacc, m_run, l_part, c, hh, nvalid);
  half_softmax_pv<D, MASK>(buf, vbase, sacc[1], 1, oacc, m_run, l_part, c, hh, nvalid);
}

// One 32-key half (kb) of a 64-key tile for one wavefront: the S^T MFMAs of
// that half, its online softmax and its P.V MFMAs (two key groups splitting
// each tile between them).
template <int D, bool MASK, typename F = NoHook>
__device__ __forceinline__ void half_tile_step(const char* buf, int kbase, int vbase, const bf16x8_t* qf,
                                               f32x16_t* oacc, float& m_run, float& l_part, float c, int hh,
                                               int nvalid, int kb, F&& after_s = F()) {
  using TG = TileGeom<D>;
  constexpr int NDC = D / 16;
  f32x16_t sacc;
#pragma unroll
  for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
  bf16x8_t ka[NDC];
  const char* kbuf = buf + kb * 32 * TG::ROWB;
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) ka[dc] = *reinterpret_cast<const bf16x8_t*>(kbuf + (kbase ^ (32 * dc)));
  __builtin_amdgcn_sched_group_barrier(0x100, NDC, 0);
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc], qf[dc], sacc, 0, 0, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, NDC, 0);
  after_s();
  half_softmax_pv<D, MASK>(buf, vbase, sacc, kb, oacc, m_run, l_part, c, hh, nvalid);
}

// The generated tokens of one wave's beams as one 32-key block on the matrix
// cores. With four query heads per kv head a wave's 32 rows are 8 beams; LDS
// row 8t + b of the block (t < 3) holds token t of beam b, K rows then V
// rows, each in the tile layout (K rows 24..31 read whatever follows and are
// masked; V rows 24..31 are not read). A row's score against key 8t + b is
// kept only for its own beam b and a token t < L.
template <int D>
__device__ __forceinline__ void token_block_step(const char* blk, const bf16x8_t* qf, f32x16_t* oacc,
                                                 float& m_run, float& l_part, float c, int own_beam, int L) {
  using TG = TileGeom<D>;
  const int lane = fresh_lane();
  const int hh = lane >> 5;
  const int kbase = k_operand_base<D>(lane), vbase = v_operand_base<D>(lane);
  constexpr int NDC = D / 16;
  f32x16_t sacc;
#pragma unroll
  for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
  bf16x8_t ka[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) ka[dc] = *reinterpret_cast<const bf16x8_t*>(blk + (kbase ^ (32 * dc)));
  __builtin_amdgcn_sched_group_barrier(0x100, NDC, 0);
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc], qf[dc], sacc, 0, 0, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, NDC, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // key 8 * (i / 4) + 4 * hh + i % 4: token i / 4 of beam 4 * hh + i % 4
    if (4 * hh + (i & 3) != own_beam || (i >> 2) >= L) sacc[i] = neg_inf();
  }
  half_softmax_pv<D, false, true>(blk + 24 * TG::ROWB - TG::TILEB, vbase, sacc, 0, oacc, m_run, l_part, c, hh, BN);
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// A buffer descriptor (base, no stride, num_records bytes, the same format
// word as the loads' other descriptors) as four scalar words.
__device__ __forceinline__ i32x4_t raw_rsrc_words(const void* base, int num_records) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4_t{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), num_records, 0x00020000};
}

// One direct HBM -> LDS load of 16 bytes per lane (buffer_load_dwordx4 with
// the lds bit) to LDS byte address `lds` (uniform), written as inline
// assembly: the compiler's wait insertion cannot tell which LDS range such a
// load writes and would wait for every one in flight before each LDS read
// of the other stage. The walks wait for these loads themselves (vmcnt) and
// publish them with a barrier. No register is written.
// NT marks the load non-temporal (chosen per call, outside the unrolled load
// sequences). The kernel streams a prompt when its workgroup is the keys'
// only reader: one row tile, and prompts of different requests disjoint.
// Measured on MI355X: streaming such keys is faster (64 distinct
// 4608-token sequences, one decode: 226 -> 201 us); where the row tiles of a
// (request, kv head) share the keys through L2 it is slower (16 requests of
// 256 beams over 16384-token prompts: 2026 -> 2153 us), and so it is for
// prompts that several requests alias (16 requests on each of 4 shared
// 4608-token ranges: 147 -> 160 us); those keep the default policy.
template <bool NT>
__device__ __forceinline__ void lds_dma16(i32x4_t rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  if constexpr (NT)
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                     :
                     : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                     : "memory", "m0");
  else
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :
                     : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                     : "memory", "m0");
}

// ---- Software-pipelined walk over full 64-key tiles (one key group) ----
//
// A wavefront works through 32-key halves. Half h's S^T MFMAs are issued
// while the probabilities of half h-1 are formed on the vector ALU (scale,
// exp2, bf16 packing, row sum), and half h-1's P.V MFMAs run while half h's
// row maxima are taken. Half h's rescale branch is taken after the first
// S^T MFMAs of half h+1 are issued (they do not depend on it), so the matrix
// core has work while the wave resolves the branch; the output it rescales
// holds every half up to h-1, and half h's probabilities, formed next, use
// the updated offset.

// K operands of one 32-key half (kb) of the tile at buf.
template <int D>
__device__ __forceinline__ void read_k_half(const char* buf, int kbase, int kb, bf16x8_t* ka) {
  using TG = TileGeom<D>;
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc)
    ka[dc] = *reinterpret_cast<const bf16x8_t*>(buf + (kbase ^ (32 * dc)) + kb * 32 * TG::ROWB);
}

// S^T of one half on the matrix cores (the first MFMA starts from zero).
template <int D>
__device__ __forceinline__ f32x16_t s_half(const bf16x8_t* ka, const bf16x8_t* qf) {
  f32x16_t sacc;
#pragma unroll
  for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc], qf[dc], sacc, 0, 0, 0);
  return sacc;
}

// Probabilities of one half (raw scores sc, offset m), packed to bf16 for
// the P.V MFMAs, and their running sum.
__device__ __forceinline__ void probs_half(const f32x16_t& sc, float c, float m, bf16x8_t* pf, float& l) {
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float p = exp2_approx(__builtin_fmaf(sc[i], c, -m));
    lsum += p;
    pf[i >> 3][i & 7] = (__bf16)p;
  }
  l += lsum;
}

// Raw row maximum of one half's scores over both lane halves.
__device__ __forceinline__ float rowmax_half(const f32x16_t& sc) {
  float mx = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, sc[i]), sc[i + 1]);
  return max_halves(fmaxf(mx, sc[15]));
}

// O^T += V^T . P^T for one half (kb) of the tile at buf.
template <int D>
__device__ __forceinline__ void pv_half(const char* buf, int vbase, int kb, const bf16x8_t* pf, f32x16_t* oacc) {
  using TG = TileGeom<D>;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const int vo = (vbase ^ (64 * db)) + (16 * (2 * kb + ch)) * TG::ROWB;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(buf + vo));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(buf + vo + 8 * TG::ROWB));
      const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[ch], oacc[db], 0, 0, 0);
    }
}

// S^T of the next half with the pending rescale decision taken after its
// first MFMAs are issued (they do not depend on it), then the rest of S^T
// beside the probabilities of the current half at the updated offset.
template <int D, typename RS>
__device__ __forceinline__ void pipe_s_rescale_probs(const char* kbuf, int kbase, int kb, const bf16x8_t* qf,
                                                     f32x16_t& sn, const f32x16_t& sc, float c, const float& m,
                                                     bf16x8_t* pf, float& l, RS&& rescale, float mx) {
  bf16x8_t ka[D / 16];
  read_k_half<D>(kbuf, kbase, kb, ka);
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[1], qf[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[2], qf[2], acc, 0, 0, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  rescale(mx);
#pragma unroll
  for (int dc = 3; dc < D / 16; ++dc) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc], qf[dc], acc, 0, 0, 0);
  probs_half(sc, c, m, pf, l);
  sn = acc;
#pragma unroll
  for (int k = 3; k < D / 16; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
  }
}

// P.V of the current half with its V^T reads, then the row maximum of the
// next half's scores (ready by then).
template <int D>
__device__ __forceinline__ float pipe_pv_then_max(const char* buf, int vbase, int kb, const bf16x8_t* pf,
                                                  f32x16_t* oacc, const f32x16_t& sn) {
  pv_half<D>(buf, vbase, kb, pf, oacc);
  const float mx = rowmax_half(sn);
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int k = 0; k < D / 16; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    if (k >= 2) __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
  }
  return mx;
}

// Wait until at most n vector-memory operations are in flight. The counter
// field needs an immediate (at most 63), so n is rounded down to a multiple
// of 8 (a smaller count only waits longer).
__device__ __forceinline__ void wait_vm_at_most(int n) {
  if (n >= 63) wait_vm<63>();
  else if (n >= 56) wait_vm<56>();
  else if (n >= 48) wait_vm<48>();
  else if (n >= 40) wait_vm<40>();
  else if (n >= 32) wait_vm<32>();
  else if (n >= 24) wait_vm<24>();
  else if (n >= 16) wait_vm<16>();
  else if (n >= 8) wait_vm<8>();
  else wait_vm<0>();
}

// Wait until at most N (if keep) or no vector-memory operations are in
// flight (keep is uniform).
template <int N>
__device__ __forceinline__ void wait_vm_keep(bool keep) {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  if (keep)
    wait_vm<N>();
  else
    wait_vm<0>();
}

// Wait until at most `ahead` tiles' loads (each `lpt` instructions per wave)
// are still in flight. The counter field needs an immediate, hence the switch.
// (The field holds at most 63; a smaller count only waits longer.)
template <int LPT>
__device__ __forceinline__ void wait_tiles(int ahead) {
  constexpr int one = LPT < 63 ? LPT : 63;
  constexpr int two = 2 * LPT < 63 ? 2 * LPT : 63;
  switch (ahead) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<one>(); break;
    default: wait_vm<two>(); break;
  }
}

constexpr int kMaxFusedTokens = 16;  // Non-Shared tokens folded into the Shared pass

// The Non-Shared stage folded into a Shared-stage wave: the beam's own
// generated tokens, gathered through its slot-table row. Lane (hh, c) holds
// head-dim halves of query row c, so a dot product needs one exchange with
// lane c + 32. With key groups, group kg takes tokens kg, kg + KG, ...
template <int D, int KG>
struct NonShared {
  static constexpr int NDC = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int NT = kMaxFusedTokens / KG;  // tokens per wave at most
  int L;  // generated tokens of the request (uniform)
  int kg;
  int tnew;  // fused append: index of the token read from knew/vnew, else -1
  const int32_t* trow;  // the slot-table row the beam's tokens come from
  const uint16_t* kp;
  const uint16_t* vp;
  const uint16_t* knew;  // this lane's parts of the beam's new K/V rows
  const uint16_t* vnew;
  int hkv;

  // Does this wave take a u-th token (token kg + KG*u)?
  __device__ __forceinline__ bool has(int u) const { return kg + KG * u < L; }
  __device__ __forceinline__ bool is_new(int u) const { return kg + KG * u == tnew; }
  __device__ __forceinline__ int slot(int u) const { return has(u) && !is_new(u) ? trow[kg + KG * u] : 0; }

  // This lane's parts of the K and V rows of token u (pool slot `sl`).
  __device__ __forceinline__ void fetch(int u, int sl, uint4* kk, uint2 (*vv)[4]) const {
    const int64_t row = (int64_t)sl * hkv * D;
    const bool nw = is_new(u);
    const uint16_t* kr = nw ? knew : kp + row;
    const uint16_t* vr = nw ? vnew : vp + row;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) kk[dc] = *reinterpret_cast<const uint4*>(kr + 16 * dc);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) vv[db][ig] = *reinterpret_cast<const uint2*>(vr + 32 * db + 8 * ig);
  }
};

// Online-softmax update with one generated token whose K/V parts are in
// registers.
template <int D>
__device__ __forceinline__ void token_update(const uint4* kk, const uint2 (*vv)[4], const bf16x8_t* qf,
                                             f32x16_t* oacc, float& m_run, float& l_part, float c, int hh) {
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  float dot = 0.f;
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
    const bf16x8_t k8 = __builtin_bit_cast(bf16x8_t, kk[dc]);
#pragma unroll
    for (int j = 0; j < 8; ++j) dot += (float)qf[dc][j] * (float)k8[j];
  }
  dot += xor32(dot);
  const float st = dot * c;
  if (st > m_run) {
    const float alpha = exp2_approx(m_run - st);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    l_part *= alpha;
    m_run = st;
  }
  const float p = exp2_approx(st - m_run);
  if (hh == 0) l_part += p;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const uint2 u = vv[db][ig];
      oacc[db][4 * ig + 0] += p * bf16_bits_to_f32(u.x & 0xffffu);
      oacc[db][4 * ig + 1] += p * __uint_as_float(u.x & 0xffff0000u);
      oacc[db][4 * ig + 2] += p * bf16_bits_to_f32(u.y & 0xffffu);
      oacc[db][4 * ig + 3] += p * __uint_as_float(u.y & 0xffff0000u);
    }
}

// Store NB column blocks of 32 (this lane's 4-float groups of one query row).
template <int NB>
__device__ __forceinline__ void store_rows(float* dst, const f32x16_t* oacc) {
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig)
      *reinterpret_cast<float4*>(dst + 32 * db + 8 * ig) =
          make_float4(oacc[db][4 * ig], oacc[db][4 * ig + 1], oacc[db][4 * ig + 2], oacc[db][4 * ig + 3]);
}

// Workgroup roles: members 0 .. p_splits-1 attend to one key range of the
// prompt each; with a.gen_member, member p_splits attends only to the beams'
// generated tokens (so that work runs beside the prompt splits instead of
// ahead of split 0). NS = LDS pipeline stages (tiles in flight + 1).
//
// Key groups (KG = 2): the NW waves form KG groups of RG = NW/KG waves; each
// group covers the same 32*RG query rows. With two LDS stages, group kg takes
// the 64-key tiles kg, kg+KG, ... of the range and each step loads KG tiles
// (one super-tile) into one stage. With four stages (which only fit for
// 64-key steps) each step loads one tile and group kg takes its 32-key half
// kg: half the work per step, three steps of loads in flight. At the end the groups' softmax states are combined through
// LDS with the log-sum-exp rule; group kg then finalizes and stores column
// blocks [kg*NDB/KG, (kg+1)*NDB/KG) of the head dim.
template <int D, int NW, int NS, int KG, bool TB = false>
__global__ __launch_bounds__(NW * 64, NW >= 8 ? 1 : 2) void shared_mfma_kernel(SharedMfmaArgs a,
                                                                               int64_t n_logical) {
  // The host pass only needs this kernel's signature for its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  using TG = TileGeom<D>;
  // Groups split tiles in halves: KG = 2 with four stages (one tile a step),
  // or KG = 4 (two tiles a step, groups 2t and 2t+1 on tile t).
  constexpr bool HALF = (KG == 2 && NS == 4) || KG == 4;
  constexpr int TPS = KG == 4 ? 2 : (HALF ? 1 : KG);  // 64-key tiles per step
  using LP = LoadPlan<D, NW, TPS>;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int RG = NW / KG;          // row groups of 32 query rows
  constexpr int NDBW = NDB / KG;       // column blocks each wave finalizes
  constexpr int ST = BN * TPS;          // keys per step
  constexpr int SBUF = TPS * TG::BUFB;  // LDS bytes per stage
  constexpr int LPT = 2 * LP::NJ;      // load instructions per super-tile per wave
  static_assert(KG == 1 || KG == 2 || KG == 4, "one, two or four key groups");
  static_assert(NDB % KG == 0, "every key group finalizes whole column blocks");
  static_assert(KG == 1 || RG * NDB * (KG - 1) * 4096 + 2 * KG * RG * 32 * 4 <= NS * SBUF,
                "the key-group exchange must fit in the stage buffers");
  // TB (four key groups, four query heads per kv head, at most three
  // generated tokens): per row group, the token block (24 K rows, 24 V rows)
  // is moved into LDS during the prompt loop by groups 0..2 (token kg each)
  // and group 3 runs it on the matrix cores after the loop. It sits behind
  // the stage buffers in the same array.
  constexpr bool LTOK = TB;
  static_assert(!TB || (NW == 8 && KG == 4 && D == 128 && NS == 2), "token block: the four-group kernel");
  constexpr int TOKRG = 2 * 24 * TG::ROWB;
  __shared__ __attribute__((aligned(1024))) char smem[NS * SBUF + (TB ? RG * TOKRG : 0)];
  char* const s_tok = smem + NS * SBUF;
  __shared__ int s_last;
  __shared__ int s_par[RG * 32 + 1];    // fused append: parents of the owned beams

  const int64_t lb64 = xcd_logical_block(blockIdx.x, gridDim.x, n_logical);
  if (lb64 < 0) return;  // uniform per workgroup
  const Shape& s = a.s;
  const int members = a.p_splits + (a.gen_member ? 1 : 0);
  // Block coordinates are workgroup-uniform; readfirstlane keeps them (and
  // everything derived from them) in scalar registers.
  const int lb = __builtin_amdgcn_readfirstlane((int)lb64);
  const int tile = __builtin_amdgcn_readfirstlane(lb % a.row_tiles);
  const int t2 = lb / a.row_tiles;
  const int member = __builtin_amdgcn_readfirstlane(t2 % members);
  const int pair = __builtin_amdgcn_readfirstlane(t2 / members);
  const int h = pair % s.Hkv;
  const int r = pair / s.Hkv;
  const int G = s.Hq / s.Hkv;
  const int M = s.B * G;
  const float c = s.scale_log2;
  const bool gen_only = a.gen_member && member == a.p_splits;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS addresses stay scalar
  const int kg = __builtin_amdgcn_readfirstlane(wave / RG);
  const int rg = wave - kg * RG;
  const int hh = lane >> 5;
  const int ql = lane & 31;

  // Query rows, the per-request values (prompt length and offset, generated
  // length) and the first slot cells are requested together, before
  // anything waits. The per-request values go through vector loads (an index
  // the compiler cannot prove uniform): as scalar loads each would wait for
  // the one before it, the scalar cache returning out of order.
  // Rows past the last query row compute on a copy of that row (their
  // columns of S^T and O^T are independent of the others) and store nothing.
  // Fused append (uniform): done by prompt split 0's workgroups (the only
  // member without a prompt split).
  const bool app = a.append != 0 && member == 0;
  const int row = tile * (RG * 32) + rg * 32 + ql;
  const bool row_ok = row < M;
  const int rowc = min(row, M - 1);
  const int bq = rowc / G;
  const int gq = rowc - bq * G;
  const int64_t qrow = ((int64_t)r * s.B + bq) * s.Hq + h * G + gq;
  // Non-Shared tokens: in the generated-token member, or (no such member) in
  // prompt split 0. They are folded in after the prompt tiles.
  const bool do_ns = a.k_pool != nullptr && (gen_only || (!a.gen_member && member == 0));
  // Slot cells read now come from this beam's row; with the fused append
  // they depend on the parent and are read once it is known.
  const bool early_slots = do_ns && !app;
  // With one workgroup per CU and registers to spare, the first NPF tokens'
  // K/V rows are requested right after the first super-tile's compute, so
  // they have landed by the end of the loop; the others are fetched after
  // the loop, the first slot cell already in hand.
  constexpr int NPF = (NS * SBUF > 80 * 1024 && NW <= 4) ? 2 : 0;
  constexpr int NSL = NPF > 0 ? NPF : 1;
  // One key group, head dim 128, two stages: the full tiles go through the
  // software-pipelined walk.
  constexpr bool PIPE = D == 128 && KG == 1 && NS == 2 && !TB && NPF == 0;
  int zv;
  __asm__ volatile("v_mov_b32 %0, 0" : "=v"(zv));
  const int Pv = a.prefix_len[r + zv];
  const int64_t poffv = a.prefix_off[r + zv];
  // Branch-free (a branch here would make the compiler wait for these reads
  // where the paths join): without Non-Shared tokens the reads go to
  // prefix_len[0], which always exists; slot cells are clamped to the row
  // and ignored beyond the length.
  const int32_t* lenp = (do_ns || app) ? a.unshared_len + r : a.prefix_len;
  const int32_t* trow = early_slots ? a.slot_table + ((int64_t)r * s.B + bq) * s.T_max : a.prefix_len;
  const int tlast = early_slots ? s.T_max - 1 : 0;
  const int lenv = lenp[zv];
  int pslot[NSL];
#pragma unroll
  for (int u = 0; u < NSL; ++u) pslot[u] = trow[min(kg + KG * u, tlast)];
  // Fused append: the request's activity flag, the row's parent and the
  // request's slot base (valid stand-in addresses otherwise).
  const bool has_act = app && a.active != nullptr;
  const uint8_t* actp = has_act ? a.active + r : reinterpret_cast<const uint8_t*>(a.prefix_len);
  const int32_t* parp = app ? a.parent + (int64_t)r * s.B + bq : a.prefix_len;
  const int64_t* sbp = app ? a.slot_base + r : a.prefix_off;
  const int actv = actp[zv];
  const int parv = parp[zv];
  const int64_t sbv = sbp[zv];
  // Token block (LTOK): for i = 0, 1 lane l moves 16-byte chunk l % 16 of
  // block row 8 kg + 4 i + l / 16, i.e. of beam bw0 + 4 i + l / 16 (clamped
  // to the request); with the fused append the beam's parent is requested
  // now.
  const bool ltok_shape = LTOK && do_ns && kg < 3;  // uniform per wave
  const int bw0 = (tile * (RG * 32) + rg * 32) / G;  // this wave's first beam (G = 4)
  auto tbeam = [&](int i) { return min(bw0 + 4 * i + (lane >> 4), s.B - 1); };
  int tref[2] = {0, 0};
  if constexpr (LTOK) {
    if (ltok_shape && app) {  // uniform
#pragma unroll
      for (int i = 0; i < 2; ++i) tref[i] = a.parent[(int64_t)r * s.B + tbeam(i)];
    }
  }
  bf16x8_t qf[NDC];
  {
    const uint16_t* qp = a.q + qrow * D + 8 * hh;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) qf[dc] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + 16 * dc));
  }

  // Per-request values are the same for the whole workgroup.
  const int P = __builtin_amdgcn_readfirstlane(Pv);
  const int64_t poff_u = ((int64_t)__builtin_amdgcn_readfirstlane((int)(poffv >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)(poffv & 0xffffffff));
  const int64_t kvbase = ((int64_t)h * s.n_ptok + poff_u) * D;
  const uint16_t* Kg = a.k_shared + kvbase;
  const uint16_t* Vg = a.v_shared + kvbase;
  const int kbeg = member * a.p_chunk;
  const int kend = min(P, kbeg + a.p_chunk);
  const int nkeys = __builtin_amdgcn_readfirstlane((!gen_only && kend > kbeg) ? kend - kbeg : 0);
  const int nsup = (nkeys + ST - 1) / ST;
  LP lp;
  lp.init(wave, lane);
  lds_char* lsm = (lds_char*)smem;
  const int prompt_bytes = P * TG::ROWB;
  // Direct HBM->LDS loads of super-tile t into its stage buffer. Buffer loads
  // address the prompt through descriptors bounded to its P_r rows, so keys
  // past the prompt read as zero (they are masked) and no load leaves it; the
  // only per-lane operand is the loop-invariant offset.
  // Key groups (one workgroup per CU): the row tiles of a (request, kv
  // head) walk the full super-tiles in rotated orders, each starting at its
  // own, so their first loads fetch different parts of the prompt from HBM
  // and every later load finds its super-tile already in L2, brought in by
  // the workgroup that started there. The last (possibly partial) super-tile
  // stays last. The softmax result does not depend on the order.
  const int rot = (KG >= 2 && nsup > 2) ? tile % (nsup - 1) : 0;
  // The loads go through lds_dma16 (the walks wait for them with explicit
  // vmcnt counts and publish them with a barrier); the refill of the other
  // stage is then no reason for the compiler to wait before this stage's
  // LDS reads.
  const i32x4_t rk_w = raw_rsrc_words(Kg, prompt_bytes);
  const i32x4_t rv_w = raw_rsrc_words(Vg, prompt_bytes);
  const bool stream = a.stream_kv != 0;  // this workgroup is its keys' only reader
  auto issue_part = [&](int t, bool do_k, bool do_v) {
    const uint32_t buf = (uint32_t)(uintptr_t)lsm + (uint32_t)((t % NS) * SBUF + wave * 1024);
    const int pt = t < nsup - 1 ? (t + rot) % (nsup - 1) : t;  // super-tile loaded at step t
    // (uniform: kept in a scalar register, the loads' scalar offset)
    const uint32_t tile_bytes = __builtin_amdgcn_readfirstlane((uint32_t)((kbeg + pt * ST) * TG::ROWB));
    auto go = [&](auto nt_c) {
      constexpr bool NT = decltype(nt_c)::value;
#pragma unroll
      for (int j = 0; j < LP::NJ; ++j)
        if (do_k) lds_dma16<NT>(rk_w, __builtin_amdgcn_readfirstlane(buf + LP::lds_off(j)), lp.k[j], tile_bytes);
#pragma unroll
      for (int j = 0; j < LP::NJ; ++j)
        if (do_v)
          lds_dma16<NT>(rv_w, __builtin_amdgcn_readfirstlane(buf + LP::lds_off(j) + TG::TILEB), lp.v[j], tile_bytes);
    };
    if (stream)
      go(std::true_type{});
    else
      go(std::false_type{});
  };
  auto issue_tile = [&](int t) { issue_part(t, true, true); };
  // The pipelined walk refills the K and V halves of a stage separately (all
  // K loads of a tile, then all V loads, so that vmcnt counts them in that
  // order).
  auto issue_asm = [&](int t, bool is_v) {  // full tile t (no rotation with one key group)
    const uint32_t base = (uint32_t)(uintptr_t)lsm + (uint32_t)((t % NS) * SBUF + wave * 1024 + (is_v ? TG::TILEB : 0));
    const uint32_t tile_bytes = __builtin_amdgcn_readfirstlane((uint32_t)((kbeg + t * ST) * TG::ROWB));
    auto go = [&](auto nt_c) {
      constexpr bool NT = decltype(nt_c)::value;
#pragma unroll
      for (int j = 0; j < LP::NJ; ++j)
        lds_dma16<NT>(is_v ? rv_w : rk_w, __builtin_amdgcn_readfirstlane(base + LP::lds_off(j)),
                      is_v ? lp.v[j] : lp.k[j], tile_bytes);
    };
    if (stream)
      go(std::true_type{});
    else
      go(std::false_type{});
  };
  NonShared<D, KG> ns;
  ns.L = early_slots ? __builtin_amdgcn_readfirstlane(lenv) : 0;  // the fused append sets it below
  ns.kg = kg;
  ns.tnew = -1;
  ns.hkv = s.Hkv;
  // The per-lane row pointers are set where the tokens are fetched (after
  // the prompt loop with the pipelined walk, whose registers are tight).
  auto set_row_ptrs = [&]() {
    ns.kp = do_ns ? a.k_pool + (int64_t)h * D + 8 * hh : a.q;
    ns.vp = do_ns ? a.v_pool + (int64_t)h * D + 4 * hh : a.q;
    ns.knew = ns.kp;
    ns.vnew = ns.vp;
    if (app) {  // uniform
      const int64_t nrow = (((int64_t)r * s.B + bq) * s.Hkv + h) * D;
      ns.knew = a.k_new + nrow + 8 * hh;
      ns.vnew = a.v_new + nrow + 4 * hh;
    }
  };
  if constexpr (!PIPE) set_row_ptrs();
  ns.trow = trow;
  uint4 pk[NPF > 0 ? NPF : 1][NDC];
  uint2 pv[NPF > 0 ? NPF : 1][NDB][4];
  // K/V rows of the first NPF tokens (missing ones read slot 0 / the first
  // query row, in bounds either way).
  auto fetch_tokens = [&]() {
#pragma unroll
    for (int u = 0; u < NPF; ++u) {
      const int sl = ns.has(u) ? pslot[u] : 0;
      ns.fetch(u, sl, pk[u], pv[u]);
    }
  };

  // Super-tiles 0 .. NS-2 go in flight next.
  int issued = 0;
#pragma unroll
  for (int t = 0; t < NS - 1; ++t) {
    if (t < nsup) {
      issue_tile(t);
      issued = t + 1;
    }
  }

  // Fused append (prompt split 0's workgroups). This workgroup owns the
  // beams whose first query row is in its row tile: it copies their new K/V
  // rows (head h) to the pool and writes its kv head's share of their
  // table_out rows. t comes from the length read above
  // (its low bits: other workgroups' arrivals only touch the bits from
  // kArrivalShift up); the workgroup arrives after its prompt loop (where
  // the workgroups of a request arrive spread out in time: same-address
  // atomics are serialized, and the round trip overlaps the token fetches),
  // and the request's last arrival, necessarily after every workgroup's
  // read, stores the new length at its end. The beam's tokens come from the
  // parent's row of table_in plus the new row for an active request with
  // room, else its own row.
  const int RPB = RG * 32;  // query rows per workgroup
  const int b_lo = (tile * RPB + G - 1) / G;
  const int nb_own = max(0, min(s.B, (tile * RPB + RPB + G - 1) / G) - b_lo);
  int t_app = 0;
  bool grow = false;
  int old_arr = 0;  // this workgroup's arrival (thread 0)
  uint4 cpv = make_uint4(0, 0, 0, 0);  // this thread's first K/V chunk to copy
  if (app) {  // uniform
    if (kg == 0 && row_ok && gq == 0) s_par[bq - b_lo] = parv;  // read after the next barrier
    t_app = __builtin_amdgcn_readfirstlane(lenv) & ((1 << kArrivalShift) - 1);
    grow = __builtin_amdgcn_readfirstlane(actv) != 0 && t_app < s.T_max;
    if (do_ns) {  // the beam's tokens in this pass: through the parent's row, the new one from k_new/v_new
      ns.L = grow ? t_app + 1 : t_app;
      ns.tnew = grow ? t_app : -1;
      ns.trow = a.slot_table + ((int64_t)r * s.B + (grow ? parv : bq)) * s.T_max;
    }
    // The first pass of the K/V copy: its source does not depend on t, so it
    // is requested now and stored right after the prompt loop.
    if (grow && tid < nb_own * 2 * (D / 8)) {
      const int bl = tid / (D / 4), pc = tid - bl * (D / 4);
      cpv = *reinterpret_cast<const uint4*>((pc < D / 8 ? a.k_new : a.v_new) +
                                            (((int64_t)r * s.B + b_lo + bl) * s.Hkv + h) * D + 8 * (pc % (D / 8)));
    }
    if constexpr (!PIPE) set_row_ptrs();
    if (do_ns) {
#pragma unroll
      for (int u = 0; u < NSL; ++u) pslot[u] = ns.slot(u);
    }
  }
  // Token block: every group holds at most one token (L <= 3); group kg < 3
  // moves token min(kg, L - 1) (a repeat is masked out), from the pool
  // through the slot table - with the fused append through the parent's
  // row, or from k_new/v_new for the new token.
  const bool ltok = LTOK && do_ns && ns.L >= 1;  // uniform
  const int tk = min(kg, ns.L - 1);
  const bool tk_new = tk == ns.tnew;
  if constexpr (LTOK) {
    if (ltok && kg < 3 && !tk_new) {  // uniform per wave
#pragma unroll
      for (int i = 0; i < 2; ++i)
        tref[i] = a.slot_table[((int64_t)r * s.B + ((app && grow) ? tref[i] : tbeam(i))) * s.T_max + tk];
    }
  }
  // The token rows go through registers (16-byte chunks, natural order) and
  // are written to LDS in the tile layout after the loop: a direct-to-LDS
  // load inside the loop would make the compiler wait for every outstanding
  // load before each step's LDS reads.
  u32x4_t tkv[2][2];  // [K, V][i]
  auto issue_tok = [&]() {
    if constexpr (LTOK) {
      if (!ltok || kg >= 3) return;  // uniform
      // bounded to the pool (or the new rows): an out-of-range slot reads zeros
      const int nrec = (int)(tk_new ? a.new_bytes : a.pool_bytes);
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(tk_new ? a.k_new : a.k_pool), (short)0, nrec, 0x00020000);
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(tk_new ? a.v_new : a.v_pool), (short)0, nrec, 0x00020000);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t row = tk_new ? ((int64_t)r * s.B + tbeam(i)) * s.Hkv + h : (int64_t)tref[i] * s.Hkv + h;
        const uint32_t off = (uint32_t)(row * TG::ROWB) + (uint32_t)((lane & 15) * 16);
        tkv[0][i] = __builtin_amdgcn_raw_buffer_load_b128(kr, (int)off, 0, 0);
        tkv[1][i] = __builtin_amdgcn_raw_buffer_load_b128(vr, (int)off, 0, 0);
      }
    }
  };
  // After the loop: lane l holds chunk l % 16 of rows 8 kg + 4 i + l / 16.
  auto store_tok = [&]() {
    if constexpr (LTOK) {
      if (!ltok || kg >= 3) return;  // uniform
      char* tK = s_tok + rg * TOKRG;
      char* tV = tK + 24 * TG::ROWB;
      const int c = lane & 15;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int j = 8 * kg + 4 * i + (lane >> 4);
        *reinterpret_cast<u32x4_t*>(tK + j * TG::ROWB + 16 * (c ^ swz_k<D>(j))) = tkv[0][i];
        *reinterpret_cast<u32x4_t*>(tV + j * TG::ROWB + 16 * (c ^ swz_v<D>(j))) = tkv[1][i];
      }
    }
  };
  // Requested at the start of the step before the last (measured faster than
  // with the first step's or the last step's loads).
  const int tok_at = max(nsup - 2, 0);


  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = neg_inf();
  float l_part = 0.f;

  // Per-lane LDS byte bases. K operand (kb, dc): key 32*kb + ql, chunk
  // 2*dc + hh, at base_k ^ (32*dc) + kb*32*ROWB.
  const int kbase = k_operand_base<D>(lane);
  // V^T operand via ds_read_b64_tr_b16 (db, cc, half j4): within each group of
  // 16 lanes, source lane i points at key 16*cc + 8*j4 + 4*hh + i/4,
  // head-dim elements 32*db + 16*(g&1) + 4*(i%4) .. +4, so result lane i
  // receives those four keys at head-dim element 32*db + 16*(g&1) + i.
  // Address: (base_v ^ (64*db)) + (16*cc + 8*j4)*ROWB.
  const int vbase = v_operand_base<D>(lane);

  // Wait for super-tile `it`, then refill the buffer super-tile it-1 used.
  // The token rows (when fetched inside the loop) follow the loads of
  // super-tile tok_after; whatever was issued after super-tile `it` may stay
  // in flight.
  int tok_after = -1;
  // Half-tile steps with two stages (one workgroup per CU) split the refill:
  // its K tiles go out here and its V tiles once the step's S^T MFMAs are
  // issued (v_pending), which spreads the LDS writes over the step. Measured
  // on MI355X: faster there, slower where two workgroups share a CU.
  int v_pending = -1;
  auto advance = [&](int it) {
    if (NPF > 0 && NS == 2 && it == 1)  // the token rows requested after tile 1's loads may stay in flight
      wait_vm<NPF * (NDC + 4 * NDB)>();
    else if (NPF > 0 && NS > 2)
      wait_vm_at_most(min(issued - 1 - it, NS - 2) * LPT + (tok_after >= it ? NPF * (NDC + 4 * NDB) : 0));
    else
      wait_tiles<LPT>(NS == 2 ? 0 : min(issued - 1 - it, NS - 2));
    __syncthreads();  // super-tile `it` landed for every wave; it-1's buffer is free
    if (it == tok_at) issue_tok();  // before the refill: nothing is in flight here
    v_pending = -1;
    if (issued < nsup) {
      if constexpr (NS == 2 && HALF) {
        issue_part(issued, true, false);
        v_pending = issued;
      } else {
        issue_tile(issued);
      }
      ++issued;
    }
  };
  auto issue_v = [&]() {
    if (v_pending >= 0) issue_part(v_pending, false, true);
  };
  if constexpr (PIPE) {
    // Full tiles through the pipelined walk. Tile t sits at stage t % 2; the
    // loads of tile t + 1 are waited for (and made visible by a barrier)
    // before its first S^T MFMAs, and tile t + 2 is requested into stage
    // t % 2 once every wave has read tile t (a second barrier). A partial
    // last tile is requested only after the walk and goes through the
    // masked step. Every tile runs the same code: the last full tile's
    // look-ahead S^T reads the other stage, which then holds the tile before
    // it (keys already seen, so its row maximum never moves the offset) and
    // whose result is dropped; one code path keeps the loop free of the
    // register copies a join of two paths costs.
    const int nfull = nkeys / BN;
    const bool pipe = nfull >= 2;  // uniform
    if (pipe) {
      const float inv_c = 1.0f / c;
      float thr = m_run * inv_c;  // raw score above which the offset moves
      auto rescale = [&](float mx) {
        if (__any(mx > thr)) {  // uniform; rare after the first half
          const float mn = fmaxf(m_run, mx * c);
          const float alpha = exp2_approx(m_run - mn);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
          l_part *= alpha;
          m_run = mn;
          thr = mn * inv_c;
        }
      };
      wait_vmem();
      __syncthreads();  // tile 0 landed for every wave
      issue_asm(1, false);  // a full tile (nfull >= 2): K, then V
      issue_asm(1, true);
      issued = 2;
      bf16x8_t pf[2];
      f32x16_t sc, sn;
      {
        bf16x8_t ka[NDC];
        read_k_half<D>(smem, kbase, 0, ka);
        sc = s_half<D>(ka, qf);
      }
      // The rescale decision of each half is applied at the start of the
      // next step (after its first S^T MFMAs); the last one, of the dropped
      // look-ahead, is dropped with it.
      float mxp = rowmax_half(sc);
      // Refills: K of tile t + 2 goes out once every wave has read K of tile
      // t (mid-tile), V of tile t + 2 once every wave has read V of tile t
      // (end of tile); each wait leaves the one younger group in flight.
      int t = 0;
      auto body = [&](auto stage_c) {
        constexpr int S = decltype(stage_c)::value;
        const char* buf = smem + S * SBUF;
        const bool next = t + 1 < nfull, next2 = t + 2 < nfull;  // uniform
        {
          // Issue priority falls as the walk advances (3 until half the tiles
          // are done, then 2, 1 and 0 past three quarters and seven eighths):
          // of the two workgroups sharing a SIMD, the one behind is issued
          // first and catches up, so both leave the CU closer together
          // instead of the younger one finishing alone at half the
          // throughput. Measured on MI355X: 16 requests of 256 beams over
          // 16384-token prompts 1987 -> 1970 us per call, 4 requests of 512
          // beams over 2048-token prompts (one round of workgroups)
          // 94.6 -> 91.7 us.
          const int rem = nfull - t;  // uniform
          if (rem * 2 > nfull) __builtin_amdgcn_s_setprio(3);
          else if (rem * 4 > nfull) __builtin_amdgcn_s_setprio(2);
          else if (rem * 8 > nfull) __builtin_amdgcn_s_setprio(1);
          else __builtin_amdgcn_s_setprio(0);
        }
        pipe_s_rescale_probs<D>(buf, kbase, 1, qf, sn, sc, c, m_run, pf, l_part, rescale, mxp);
        mxp = pipe_pv_then_max<D>(buf, vbase, 0, pf, oacc, sn);
        sc = sn;
        // K of tile t + 1 landed (its V may still be in flight)
        wait_vm_keep<LP::NJ>(next);
        __syncthreads();
        if (next2) issue_asm(t + 2, false);
        // half 1: S^T of the next tile's first half (the other stage; for
        // the last tile that stage holds keys already seen, result dropped)
        pipe_s_rescale_probs<D>(smem + (S ^ 1) * SBUF, kbase, 0, qf, sn, sc, c, m_run, pf, l_part, rescale, mxp);
        mxp = pipe_pv_then_max<D>(buf, vbase, 1, pf, oacc, sn);
        // V of tile t + 1 landed (K of tile t + 2 may still be in flight)
        wait_vm_keep<LP::NJ>(next2);
        __syncthreads();
        if (next2) {
          issue_asm(t + 2, true);
          issued = t + 3;
        }
        sc = sn;
        ++t;
      };
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      while (t + 1 < nfull) {
        body(I0{});
        body(I1{});
      }
      if (t < nfull) body(I0{});
      __builtin_amdgcn_s_setprio(0);  // the default again for the rest of the kernel
    }
    // Without two full tiles, or for the partial last tile: the masked step
    // (its loads requested now when the walk left them out).
    if (!pipe) wait_vmem();  // (the walk waited already) the query rows have landed
    for (int it = pipe ? nfull : 0; it < nsup; ++it) {
      if (pipe && issued <= it) {
        issue_tile(it);
        issued = it + 1;
      }
      advance(it);
      const int nv = min(nkeys - it * BN, BN);
      const char* buf = smem + (it % NS) * SBUF;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {  // one half at a time: few registers
        if (nv <= 32 * kb) break;  // uniform
        bf16x8_t ka[NDC];
        read_k_half<D>(buf, kbase, kb, ka);
        f32x16_t sacc = s_half<D>(ka, qf);
        half_softmax_pv<D, true>(buf, vbase, sacc, kb, oacc, m_run, l_part, c, hh, nv);
      }
    }
  } else {
  // The query rows (and the prologue's other register loads) have landed:
  // with that wait visible to the compiler it puts none of its own inside
  // the loop. (Two stages: the first step waits for everything anyway.)
  wait_vmem();
  // This wave's tile of super-tile `it` sits at stage (it % NS), slot kg.
  for (int it = 0; it + 1 < nsup; ++it) {  // full super-tiles
    // Issue priority falls with the walk's progress, as in the pipelined walk.
    // Measured on MI355X (64 single-beam requests on 4 shared 4608-token
    // prompts): 151.4 -> 146.0 us per call; distinct prompts unchanged.
    if constexpr (NW == 4) {
      const int rem = nsup - it;  // uniform
      if (rem * 2 > nsup) __builtin_amdgcn_s_setprio(3);
      else if (rem * 4 > nsup) __builtin_amdgcn_s_setprio(2);
      else if (rem * 8 > nsup) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    advance(it);
    if constexpr (HALF)
      half_tile_step<D, false>(smem + (it % NS) * SBUF + (kg >> 1) * (TPS - 1) * TG::BUFB, kbase, vbase, qf,
                               oacc, m_run, l_part, c, hh, BN, TPS == 2 ? (kg & 1) : kg, issue_v);
    else
      tile_step<D, false>(smem + (it % NS) * SBUF + kg * TG::BUFB, kbase, vbase, qf, oacc, m_run, l_part, c,
                          hh, BN, issue_v);
    if (NPF > 0 && it == 0) {
      __asm__ volatile("" ::: "memory");  // keep these loads after the tiles issued so far
      fetch_tokens();
      tok_after = issued - 1;
    }
  }
  if constexpr (NW == 4) __builtin_amdgcn_s_setprio(0);
  if (NPF > 0 && nsup <= 1) fetch_tokens();
  if (nsup > 0) {  // the last super-tile: this wave's tile may be partial or empty
    const int it = nsup - 1;
    advance(it);
    if constexpr (HALF) {
      const int sub = TPS == 2 ? (kg >> 1) : 0, half = TPS == 2 ? (kg & 1) : kg;
      const int nv = nkeys - (it * TPS + sub) * BN;  // valid keys of this group's tile
      if (nv > 32 * half)
        half_tile_step<D, true>(smem + (it % NS) * SBUF + sub * TG::BUFB, kbase, vbase, qf, oacc, m_run, l_part,
                                c, hh, min(nv, BN), half);
    } else {
      const int nv = nkeys - (it * KG + kg) * BN;
      if (nv > 0)
        tile_step<D, true>(smem + (it % NS) * SBUF + kg * TG::BUFB, kbase, vbase, qf, oacc, m_run, l_part, c,
                           hh, min(nv, BN));
    }
  }
  }  // !PIPE
  if constexpr (PIPE) set_row_ptrs();

  if (nsup == 0) issue_tok();
  wait_vmem();  // every tile load has landed before the stage buffers are reused
  store_tok();
  if (ltok) __syncthreads();  // the token block is complete in LDS; the stage buffers are free

  // Fused append writes: the first K/V chunk (loaded in the prologue) is
  // stored now; the first table cells are requested before the tokens' rows
  // (one round trip for both) and stored after them; further passes follow.
  constexpr int NTH = NW * 64;
  constexpr int CH = D / 8;                      // 16-byte chunks per K (or V) row
  const int n_cp = grow ? nb_own * 2 * CH : 0;   // K/V chunks to copy
  const int tc = grow ? t_app + 1 : t_app;       // table cells per owned row
  // The kv heads' workgroups share the owned rows' cells: head h copies
  // columns [tj0, tj0 + tcw) (long rows are then no single workgroup's tail).
  const int tj0 = (int)((int64_t)h * tc / s.Hkv);
  const int tcw = (int)((int64_t)(h + 1) * tc / s.Hkv) - tj0;
  const int n_tb = app ? nb_own * tcw : 0;
  const int64_t sb_new = sbv + (int64_t)t_app * s.B;  // slot of beam 0's new row
  auto cp_src = [&](int i) {
    const int bl = i / (2 * CH), pc = i - bl * (2 * CH);
    const uint16_t* base = pc < CH ? a.k_new : a.v_new;
    return reinterpret_cast<const uint4*>(base + (((int64_t)r * s.B + b_lo + bl) * s.Hkv + h) * D + 8 * (pc % CH));
  };
  auto cp_dst = [&](int i) {
    const int bl = i / (2 * CH), pc = i - bl * (2 * CH);
    uint16_t* base = pc < CH ? a.k_pool_out : a.v_pool_out;
    return reinterpret_cast<uint4*>(base + ((sb_new + b_lo + bl) * s.Hkv + h) * D + 8 * (pc % CH));
  };
  auto tb_val = [&](int i) {  // table_out cell i of this head's share of the owned rows
    const int bl = i / tcw, j = tj0 + (i - bl * tcw);
    if (j == t_app) return (int32_t)(sb_new + b_lo + bl);
    const int src = grow ? s_par[bl] : b_lo + bl;
    return a.slot_table[((int64_t)r * s.B + src) * s.T_max + j];
  };
  auto tb_dst = [&](int i) {
    const int bl = i / tcw, j = tj0 + (i - bl * tcw);
    return a.table_out + ((int64_t)r * s.B + b_lo + bl) * s.T_max + j;
  };
  int32_t tbv = 0;
  if (app) {  // uniform
    if (tid < n_cp) *cp_dst(tid) = cpv;
    if (tid == 0) {
      // Two-level arrival (same-address atomics serialize): the row tiles of
      // (request, kv head) count on its own counter, which wraps back to zero;
      // the last of them arrives for the pair on the request's length.
      const unsigned n1 = __builtin_amdgcn_atomic_inc32(a.counters + pair, (unsigned)(a.row_tiles - 1),
                                                        __ATOMIC_RELAXED, "agent");
      if (n1 == (unsigned)(a.row_tiles - 1))
        old_arr = atomicAdd(a.ulen_rw + r, 1 << kArrivalShift);
      else
        old_arr = -1;  // not the pair's last
    }
    if (nsup == 0) __syncthreads();  // no loop barrier since the parents went to LDS
    if (tid < n_tb) tbv = tb_val(tid);
  }

  // The Non-Shared tokens: prefetched ones first, then the rest one at a time
  // with the next slot index in flight beside each token's K/V rows.
#pragma unroll
  for (int u = 0; u < NPF; ++u)
    if (ns.has(u)) token_update<D>(pk[u], pv[u], qf, oacc, m_run, l_part, c, hh);
  if constexpr (TB) {
    if (ltok && kg == 3)  // uniform
      token_block_step<D>(s_tok + rg * TOKRG, qf, oacc, m_run, l_part, c,
                          (tile * (RG * 32) + rg * 32 + (fresh_lane() & 31)) / G - bw0, ns.L);
  } else if (ns.has(NPF)) {
    int sl = NPF == 0 ? pslot[0] : ns.slot(NPF);
    for (int u = NPF; u < NonShared<D, KG>::NT && ns.has(u); ++u) {
      uint4 kk[NDC];
      uint2 vv[NDB][4];
      ns.fetch(u, sl, kk, vv);
      sl = ns.slot(u + 1);
      token_update<D>(kk, vv, qf, oacc, m_run, l_part, c, hh);
    }
  }

  if (app) {  // uniform
    if (tid < n_tb) *tb_dst(tid) = tbv;
    for (int i = tid + NTH; i < n_cp; i += NTH) *cp_dst(i) = *cp_src(i);
    for (int i0 = tid + NTH; i0 < n_tb; i0 += 4 * NTH) {  // four cells in flight per thread
      int32_t v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = i0 + k * NTH < n_tb ? tb_val(i0 + k * NTH) : 0;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (i0 + k * NTH < n_tb) *tb_dst(i0 + k * NTH) = v[k];
    }
    if (tid == 0 && old_arr >= 0 && (old_arr >> kArrivalShift) == a.arrivals - 1)
      a.ulen_rw[r] = grow ? t_app + 1 : t_app;
  }

  float l_tot = sum_halves(l_part);
  // own[j]: column block kg*NDBW + j of this wave's 32 rows, combined over
  // the key groups. Each group hands every other group the column blocks
  // that group finalizes (KG - 1 slots per block), then merges the ones it
  // owns with the log-sum-exp rule.
  f32x16_t own[NDBW];
  if constexpr (KG == 1) {
#pragma unroll
    for (int j = 0; j < NDB; ++j) own[j] = oacc[j];
  } else {
    float4* xo = reinterpret_cast<float4*>(smem);  // [RG][NDB][KG-1][4][64] float4
    float* xm = reinterpret_cast<float*>(smem + RG * NDB * (KG - 1) * 4096);
    float* xl = xm + KG * RG * 32;
    auto slot = [&](int db, int src) {  // exchange slot of block db from group src
      const int owner = db / NDBW;
      return (rg * NDB + db) * (KG - 1) + (src < owner ? src : src - 1);
    };
    // Every wave is done reading the stage buffers. (With the token block the
    // barrier after the loop already said so: the block reads only its own
    // LDS, so the other groups write their exchange data while it runs.)
    if (!(TB && ltok)) __syncthreads();
    if (hh == 0) {
      xm[(kg * RG + rg) * 32 + ql] = m_run;
      xl[(kg * RG + rg) * 32 + ql] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      if (db / NDBW == kg) continue;  // uniform: this group's own block
      const int sl = slot(db, kg);
#pragma unroll
      for (int ig = 0; ig < 4; ++ig)
        xo[(sl * 4 + ig) * 64 + lane] =
            make_float4(oacc[db][4 * ig], oacc[db][4 * ig + 1], oacc[db][4 * ig + 2], oacc[db][4 * ig + 3]);
    }
    __syncthreads();
    float mg[KG], lg[KG];
    float mn = neg_inf();
#pragma unroll
    for (int g = 0; g < KG; ++g) {
      mg[g] = xm[(g * RG + rg) * 32 + ql];
      lg[g] = xl[(g * RG + rg) * 32 + ql];
      mn = fmaxf(mn, mg[g]);
    }
    float ag[KG];
    float lsum = 0.f;
#pragma unroll
    for (int g = 0; g < KG; ++g) {
      ag[g] = mg[g] == neg_inf() ? 0.f : exp2_approx(mg[g] - mn);
      lsum += lg[g] * ag[g];
    }
    l_tot = lsum;
    m_run = mn;
    // this wave's own blocks: select them out of oacc (kg is only known at
    // run time; a select chain keeps oacc in registers)
#pragma unroll
    for (int j = 0; j < NDBW; ++j) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = oacc[j][i];
#pragma unroll
        for (int g = 1; g < KG; ++g) v = kg == g ? oacc[g * NDBW + j][i] : v;
        own[j][i] = v;
      }
    }
    float aself = ag[0];
#pragma unroll
    for (int g = 1; g < KG; ++g) aself = kg == g ? ag[g] : aself;
#pragma unroll
    for (int j = 0; j < NDBW; ++j) {
#pragma unroll
      for (int i = 0; i < 16; ++i) own[j][i] *= aself;
      const int db = kg * NDBW + j;
#pragma unroll
      for (int g = 0; g < KG; ++g) {
        if (g == kg) continue;  // uniform
        const int sl = slot(db, g);
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const float4 v = xo[(sl * 4 + ig) * 64 + lane];
          own[j][4 * ig + 0] += v.x * ag[g];
          own[j][4 * ig + 1] += v.y * ag[g];
          own[j][4 * ig + 2] += v.z * ag[g];
          own[j][4 * ig + 3] += v.w * ag[g];
        }
      }
    }
  }
  const int dcol = 32 * NDBW * kg;  // first head-dim column this wave finalizes
  const bool writes_lse = kg == 0 && hh == 0;

  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const float lse_here = l_tot > 0.f ? (m_run + log2_approx(l_tot)) * kLn2 : neg_inf();
#pragma unroll
  for (int j = 0; j < NDBW; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) own[j][i] *= inv;

  if (a.mode == kModeFinal) {
    if (!row_ok) return;
    store_rows<NDBW>(a.out.o + qrow * D + dcol + 4 * hh, own);
    if (a.out.lse && writes_lse) a.out.lse[qrow] = lse_here;
    return;
  }
  if (a.mode == kModePartial) {
    const int64_t part = a.out.part_base + member;
    if (!row_ok) return;
    store_rows<NDBW>(a.part_o + (part * a.part_stride + qrow) * D + dcol + 4 * hh, own);
    if (writes_lse) a.part_lse[part * a.part_stride + qrow] = lse_here;
    return;
  }

  // kModeFixup: publish this member's partial (agent-coherent), count arrivals.
  const int64_t rows = a.part_stride;
  const int obase = (int)((qrow * D + dcol + 4 * hh) * 4);
  {
    const __amdgpu_buffer_rsrc_t ro = coherent_rsrc(a.part_o + (int64_t)member * rows * D, rows * D);
    const __amdgpu_buffer_rsrc_t rl = coherent_rsrc(a.part_lse + (int64_t)member * rows, rows);
    if (row_ok) {
#pragma unroll
      for (int j = 0; j < NDBW; ++j)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const float4 v = make_float4(own[j][4 * ig], own[j][4 * ig + 1], own[j][4 * ig + 2], own[j][4 * ig + 3]);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), ro,
                                                 obase + (32 * j + 8 * ig) * 4, 0, kCoherent);
        }
      if (writes_lse)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, lse_here), rl, (int)(qrow * 4), 0,
                                              kCoherent);
    }
  }
  // Publish: every thread's partial stores are released at agent scope (the
  // members of a group may run on different XCDs, each with its own L2)
  // before the workgroup barrier, and the arrival is an acquire-release
  // agent-scope atomic; the last arrival acquires at agent scope before it
  // reads the partials back.
  wait_vmem();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __builtin_amdgcn_atomic_inc32(a.counters + (int64_t)pair * a.row_tiles + tile,
                                                       (unsigned)(members - 1), __ATOMIC_ACQ_REL, "agent");
    s_last = (old == (unsigned)(members - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last || !row_ok) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // Last arrival: combine every member's partial, always in member order, so
  // the result does not depend on which workgroup arrived last. Pass 1 finds
  // the largest lse; pass 2 sums the weighted outputs (independent loads).
  float lmax = neg_inf();
  for (int sp = 0; sp < members; ++sp) {
    const __amdgpu_buffer_rsrc_t rl = coherent_rsrc(a.part_lse + (int64_t)sp * rows, rows);
    lmax = fmaxf(lmax, __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, (int)(qrow * 4), 0, kCoherent)));
  }
#pragma unroll
  for (int j = 0; j < NDBW; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) own[j][i] = 0.f;
  float wsum = 0.f;
  if (lmax != neg_inf()) {
    for (int sp = 0; sp < members; ++sp) {
      const __amdgpu_buffer_rsrc_t ro = coherent_rsrc(a.part_o + (int64_t)sp * rows * D, rows * D);
      const __amdgpu_buffer_rsrc_t rl = coherent_rsrc(a.part_lse + (int64_t)sp * rows, rows);
      const float lo = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, (int)(qrow * 4), 0, kCoherent));
      const float w = exp2_approx((lo - lmax) * kLog2e);  // empty member: exp2(-inf) = 0
      wsum += w;
#pragma unroll
      for (int j = 0; j < NDBW; ++j)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const float4 v = __builtin_bit_cast(
              float4, __builtin_amdgcn_raw_buffer_load_b128(ro, obase + (32 * j + 8 * ig) * 4, 0, kCoherent));
          if (w != 0.f) {
            own[j][4 * ig + 0] += w * v.x;
            own[j][4 * ig + 1] += w * v.y;
            own[j][4 * ig + 2] += w * v.z;
            own[j][4 * ig + 3] += w * v.w;
          }
        }
    }
  }
  const float winv = wsum > 0.f ? 1.0f / wsum : 0.f;
#pragma unroll
  for (int j = 0; j < NDBW; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) own[j][i] *= winv;
  store_rows<NDBW>(a.out.o + qrow * D + dcol + 4 * hh, own);
  if (a.out.lse && writes_lse) a.out.lse[qrow] = wsum > 0.f ? lmax + log2_approx(wsum) * kLn2 : neg_inf();
#endif
}

template <int D, int NW, int KG>
hipError_t launch_dwk(const SharedMfmaArgs& a, int64_t grid, int64_t n_logical, hipStream_t st) {
  if constexpr (KG != 4) {
    if (a.stages == 4) {
      hipLaunchKernelGGL((shared_mfma_kernel<D, NW, 4, KG>), dim3((unsigned)grid), dim3(NW * 64), 0, st, a,
                         n_logical);
      return hipGetLastError();
    }
  }
  if constexpr (D == 128 && NW == 8 && KG == 4) {
    if (a.token_block) {
      hipLaunchKernelGGL((shared_mfma_kernel<D, NW, 2, KG, true>), dim3((unsigned)grid), dim3(NW * 64), 0, st, a,
                         n_logical);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((shared_mfma_kernel<D, NW, 2, KG>), dim3((unsigned)grid), dim3(NW * 64), 0, st, a, n_logical);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const SharedMfmaArgs& a, hipStream_t st) {
  const int members = a.p_splits + (a.gen_member ? 1 : 0);
  const int64_t n_logical = (int64_t)a.s.R * a.s.Hkv * members * a.row_tiles;
  if (n_logical == 0) return hipSuccess;
  const int64_t grid = (n_logical + 7) / 8 * 8;
  if (a.key_groups == 4) {
    if constexpr (D == 128) {
      if (a.waves == 4) return launch_dwk<D, 4, 4>(a, grid, n_logical, st);
      return launch_dwk<D, 8, 4>(a, grid, n_logical, st);
    }
    return hipErrorInvalidValue;
  }
  if (a.key_groups == 2) {
    switch (a.waves) {
      case 2: return launch_dwk<D, 2, 2>(a, grid, n_logical, st);
      case 4: return launch_dwk<D, 4, 2>(a, grid, n_logical, st);
      default: return launch_dwk<D, 8, 2>(a, grid, n_logical, st);
    }
  }
  switch (a.waves) {
    case 1: return launch_dwk<D, 1, 1>(a, grid, n_logical, st);
    case 2: return launch_dwk<D, 2, 1>(a, grid, n_logical, st);
    default: return launch_dwk<D, 4, 1>(a, grid, n_logical, st);
  }
}

}  // namespace

hipError_t launch_shared_mfma(const SharedMfmaArgs& a, hipStream_t st) {
  return a.s.D == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace xattn

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
// K/V tiles (64 keys) move HBM -> LDS with global_load_lds_dwordx4 (no
// register staging), double-buffered so tile i+1 is in flight while tile i is
// computed.
//
// Online softmax with a lazy rescale: the exponent offset only moves when a
// tile's max exceeds it by more than 8 (log2 units), which keeps every
// probability <= 256 and skips most output rescales; the result is exact
// either way because the final division uses the same offset.
//
// Non-Shared part (prompt split 0 only, when fused): the beam's own generated
// tokens, gathered through its slot-table row, initialise the softmax state
// while the first K/V tile is in flight.
//
// Prompt splits: with p_splits > 1 and mode FIXUP, every split writes its
// partial (normalized O, lse) to the workspace, and the last workgroup of a
// (request, kv head, row tile) to arrive - found with a wrapping atomic
// counter that returns to zero - merges all partials with the log-sum-exp
// rule and writes the final output. In mode PARTIAL each split only writes its
// partial slot for a later reduction.
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

// Per-lane byte offsets (within a tile) of the global chunks this lane loads
// for each of its direct-load instructions j (instruction index
// i = wave + NW*j): K then V. Loop-invariant.
template <int D, int NW>
struct LoadPlan {
  static constexpr int NJ = TileGeom<D>::NINST / NW;
  uint32_t k[NJ];
  uint32_t v[NJ];
  __device__ __forceinline__ void init(int wave, int lane) {
    using TG = TileGeom<D>;
    const int kin = lane / TG::NCH;
    const int pos = lane % TG::NCH;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int key = (wave + NW * j) * TG::KPI + kin;
      k[j] = (uint32_t)(key * TG::ROWB + (pos ^ swz_k<D>(key)) * 16);
      v[j] = (uint32_t)(key * TG::ROWB + (pos ^ swz_v<D>(key)) * 16);
    }
  }
};

typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ void wait_vmem() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Split partials that one workgroup hands to another are written and read
// with agent-coherent buffer accesses (cache policy sc1, what agent-scope
// atomic loads/stores use), so no cache-wide flush or invalidate is needed:
// writers wait for their stores to complete, then bump a relaxed agent-scope
// counter; the last arrival reads the partials back with the same policy.
constexpr int kCoherent = 16;  // sc1
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const float* base, int64_t floats) {
  const int64_t bytes = floats * 4;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0,
                                           (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff), 0x00020000);
}

// Online-softmax update for one 32-key half of a tile (S^T block `sb`, the
// 16 scores this lane holds for its query column), followed by that half's
// P.V MFMAs. Processing the halves separately lets the vector-ALU softmax of
// one half overlap the matrix-core work of the other.
template <int D, bool MASK>
__device__ __forceinline__ void half_softmax_pv(const char* buf, int vbase, f32x16_t& sb, int kb,
                                                f32x16_t* oacc, float& m_run, float& l_part, float c,
                                                int hh, int nvalid) {
  using TG = TileGeom<D>;
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
  mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;
  if (__any(mx > m_run + 8.0f)) {
    const float mn = fmaxf(m_run, mx);
    const float alpha = exp2_approx(m_run - mn);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    l_part *= alpha;
    m_run = mn;
  }
  bf16x8_t pf[2];
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float p = exp2_approx(__builtin_fmaf(sb[i], c, -m_run));
    lsum += p;
    pf[i >> 3][i & 7] = (__bf16)p;
  }
  l_part += lsum;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const int vo = (vbase ^ (64 * db)) + (16 * (2 * kb + ch)) * TG::ROWB;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(buf + vo));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(buf + vo + 8 * TG::ROWB));
      const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[ch], oacc[db], 0, 0, 0);
    }
}

// One 64-key tile for one wavefront (32 query rows): S^T = K.Q^T on MFMA for
// both 32-key halves, then per half the online softmax and O^T += V^T.P^T.
// MASK: the tile holds only `nvalid` keys (the last tile of a range).
template <int D, bool MASK>
__device__ __forceinline__ void tile_step(const char* buf, int kbase, int vbase, const bf16x8_t* qf,
                                          f32x16_t* oacc, float& m_run, float& l_part, float c,
                                          int hh, int nvalid) {
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
  half_softmax_pv<D, MASK>(buf, vbase, sacc[0], 0, oacc, m_run, l_part, c, hh, nvalid);
  half_softmax_pv<D, MASK>(buf, vbase, sacc[1], 1, oacc, m_run, l_part, c, hh, nvalid);
}

// Wait until at most `ahead` tiles' loads (each `lpt` instructions per wave)
// are still in flight. The counter field needs an immediate, hence the switch.
// (The field holds at most 63; a smaller count only waits longer.)
template <int LPT>
__device__ __forceinline__ void wait_tiles(int ahead) {
  constexpr int one = LPT < 63 ? LPT : 63;
  constexpr int two = 2 * LPT < 63 ? 2 * LPT : 63;
  switch (ahead) {
    case 0: __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(one) : "memory"); break;
    default: __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(two) : "memory"); break;
  }
}

constexpr int kMaxFusedTokens = 16;  // Non-Shared tokens folded into the Shared pass

// Online-softmax update with the beam's own generated tokens (the Non-Shared
// stage): slot indices are fetched first, then each token costs one round
// trip for its K and V rows. Lane (hh, c) holds head-dim halves of query row
// c, so the dot product needs one exchange with lane c + 32.
template <int D>
__device__ __forceinline__ void nonshared_update(const SharedMfmaArgs& a, int r, int h, int bq,
                                                 const bf16x8_t* qf, f32x16_t* oacc, float& m_run,
                                                 float& l_part, float c, int hh) {
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  const Shape& s = a.s;
  const int L = __builtin_amdgcn_readfirstlane(a.unshared_len[r]);
  const int32_t* trow = a.slot_table + ((int64_t)r * s.B + bq) * s.T_max;
  int slots[kMaxFusedTokens];
#pragma unroll
  for (int t = 0; t < kMaxFusedTokens; ++t) slots[t] = t < L ? trow[t] : 0;
#pragma unroll
  for (int t = 0; t < kMaxFusedTokens; ++t) {
    if (t >= L) break;
    const int64_t row = ((int64_t)slots[t] * s.Hkv + h) * D;
    const uint16_t* kp = a.k_pool + row + 8 * hh;
    const uint16_t* vp = a.v_pool + row + 4 * hh;
    uint4 kk[NDC];
    uint2 vv[NDB][4];
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) kk[dc] = *reinterpret_cast<const uint4*>(kp + 16 * dc);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) vv[db][ig] = *reinterpret_cast<const uint2*>(vp + 32 * db + 8 * ig);
    float dot = 0.f;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      const bf16x8_t k8 = __builtin_bit_cast(bf16x8_t, kk[dc]);
#pragma unroll
      for (int j = 0; j < 8; ++j) dot += (float)qf[dc][j] * (float)k8[j];
    }
    dot += __shfl_xor(dot, 32);
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
}

template <int D>
__device__ __forceinline__ void store_rows(float* dst, const f32x16_t* oacc) {
  constexpr int NDB = D / 32;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig)
      *reinterpret_cast<float4*>(dst + 32 * db + 8 * ig) =
          make_float4(oacc[db][4 * ig], oacc[db][4 * ig + 1], oacc[db][4 * ig + 2], oacc[db][4 * ig + 3]);
}

// Workgroup roles: members 0 .. p_splits-1 attend to one key range of the
// prompt each; with a.gen_member, member p_splits attends only to the beams'
// generated tokens (so that work runs beside the prompt splits instead of
// ahead of split 0). NS = LDS pipeline stages (tiles in flight + 1).
template <int D, int NW, int NS>
__global__ __launch_bounds__(NW * 64, 2) void shared_mfma_kernel(SharedMfmaArgs a, int64_t n_logical) {
  // The host pass only needs this kernel's signature for its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  using TG = TileGeom<D>;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int LPT = 2 * LoadPlan<D, NW>::NJ;  // load instructions per tile per wave
  __shared__ __attribute__((aligned(1024))) char smem[NS * TG::BUFB];
  __shared__ int s_last;

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
  const int wave = tid >> 6;
  const int hh = lane >> 5;
  const int ql = lane & 31;

  // Per-request values are the same for the whole workgroup.
  const int P = __builtin_amdgcn_readfirstlane(a.prefix_len[r]);
  const int64_t poff = a.prefix_off[r];
  const int64_t poff_u = ((int64_t)__builtin_amdgcn_readfirstlane((int)(poff >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)(poff & 0xffffffff));
  const int64_t kvbase = ((int64_t)h * s.n_ptok + poff_u) * D;
  const uint16_t* Kg = a.k_shared + kvbase;
  const uint16_t* Vg = a.v_shared + kvbase;
  const int kbeg = member * a.p_chunk;
  const int kend = min(P, kbeg + a.p_chunk);
  const int nkeys = __builtin_amdgcn_readfirstlane((!gen_only && kend > kbeg) ? kend - kbeg : 0);
  const int nfull = nkeys / BN;
  const int tail = nkeys - nfull * BN;
  const int ntiles = nfull + (tail > 0 ? 1 : 0);
  LoadPlan<D, NW> lp;
  lp.init(wave, lane);
  lds_char* lsm = (lds_char*)smem;
  const int prompt_bytes = P * TG::ROWB;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)Kg, (short)0, prompt_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)Vg, (short)0, prompt_bytes, 0x00020000);
  // Direct HBM->LDS loads of tile t into its stage buffer. Buffer loads
  // address the prompt through descriptors bounded to its P_r rows, so keys
  // past the prompt read as zero (they are masked) and no load leaves it; the
  // only per-lane operand is the loop-invariant offset.
  auto issue_tile = [&](int t) {
    lds_char* buf = lsm + (t % NS) * TG::BUFB;
    const uint32_t tile_bytes = (uint32_t)((kbeg + t * BN) * TG::ROWB);
#pragma unroll
    for (int j = 0; j < LoadPlan<D, NW>::NJ; ++j) {
      const int i = wave + NW * j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, buf + i * 1024, 16, lp.k[j], tile_bytes, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, buf + TG::TILEB + i * 1024, 16, lp.v[j], tile_bytes, 0, 0);
    }
  };
  // Tiles 0 .. NS-2 go in flight before anything else.
  int issued = 0;
#pragma unroll
  for (int t = 0; t < NS - 1; ++t) {
    if (t < ntiles) {
      issue_tile(t);
      issued = t + 1;
    }
  }

  const int row = tile * (NW * 32) + wave * 32 + ql;
  const bool row_ok = row < M;
  const int bq = row_ok ? row / G : 0;
  const int gq = row_ok ? row - bq * G : 0;
  const int64_t qrow = ((int64_t)r * s.B + bq) * s.Hq + h * G + gq;

  bf16x8_t qf[NDC];
  {
    const uint16_t* qp = a.q + qrow * D + 8 * hh;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (row_ok) u = *reinterpret_cast<const uint4*>(qp + 16 * dc);
      qf[dc] = __builtin_bit_cast(bf16x8_t, u);
    }
  }

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = neg_inf();
  float l_part = 0.f;

  // Non-Shared tokens: in the generated-token member, or (no such member) in
  // prompt split 0 while its first tiles are in flight.
  if (a.k_pool != nullptr && (gen_only || (!a.gen_member && member == 0)))
    nonshared_update<D>(a, r, h, bq, qf, oacc, m_run, l_part, c, hh);

  // Per-lane LDS byte bases. K operand (kb, dc): key 32*kb + ql, chunk
  // 2*dc + hh, at base_k ^ (32*dc) + kb*32*ROWB.
  int kbase;
  {
    const int f = swz_k<D>(ql);
    kbase = ql * TG::ROWB + 16 * (hh ^ (f & 1)) + 32 * (f >> 1);
  }
  // V^T operand via ds_read_b64_tr_b16 (db, cc, half j4): within each group of
  // 16 lanes, source lane i points at key 16*cc + 8*j4 + 4*hh + i/4,
  // head-dim elements 32*db + 16*(g&1) + 4*(i%4) .. +4, so result lane i
  // receives those four keys at head-dim element 32*db + 16*(g&1) + i.
  // Address: (base_v ^ (64*db)) + (16*cc + 8*j4)*ROWB.
  const int g16 = lane >> 4, i16 = lane & 15;
  int vbase;
  {
    const int e = i16 >> 2;
    const int key0 = 4 * hh + e;
    const int x = 2 * (g16 & 1) + ((i16 & 3) >> 1);
    vbase = TG::TILEB + key0 * TG::ROWB + 16 * (x ^ swz_v<D>(key0)) + (i16 & 1) * 8;
  }

  // Wait for tile `it`, then refill the buffer tile it-1 used.
  auto advance = [&](int it) {
    wait_tiles<LPT>(min(issued - 1 - it, NS - 2));
    __syncthreads();  // tile `it` landed for every wave; tile it-1's buffer is free
    if (issued < ntiles) {
      issue_tile(issued);
      ++issued;
    }
  };
  for (int it = 0; it < nfull; ++it) {
    advance(it);
    tile_step<D, false>(smem + (it % NS) * TG::BUFB, kbase, vbase, qf, oacc, m_run, l_part, c, hh, BN);
  }
  if (tail > 0) {  // the last, partial tile of the range
    advance(nfull);
    tile_step<D, true>(smem + (nfull % NS) * TG::BUFB, kbase, vbase, qf, oacc, m_run, l_part, c, hh, tail);
  }

  const float l_tot = l_part + __shfl_xor(l_part, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const float lse_here = l_tot > 0.f ? (m_run + log2_approx(l_tot)) * kLn2 : neg_inf();
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] *= inv;

  if (a.mode == kModeFinal) {
    if (!row_ok) return;
    store_rows<D>(a.out.o + qrow * D + 4 * hh, oacc);
    if (a.out.lse && hh == 0) a.out.lse[qrow] = lse_here;
    return;
  }
  if (a.mode == kModePartial) {
    const int64_t part = a.out.part_base + member;
    if (!row_ok) return;
    store_rows<D>(a.part_o + (part * a.part_stride + qrow) * D + 4 * hh, oacc);
    if (hh == 0) a.part_lse[part * a.part_stride + qrow] = lse_here;
    return;
  }

  // kModeFixup: publish this member's partial (agent-coherent), count arrivals.
  const int64_t rows = a.part_stride;
  const int obase = (int)((qrow * D + 4 * hh) * 4);
  {
    const __amdgpu_buffer_rsrc_t ro = coherent_rsrc(a.part_o + (int64_t)member * rows * D, rows * D);
    const __amdgpu_buffer_rsrc_t rl = coherent_rsrc(a.part_lse + (int64_t)member * rows, rows);
    if (row_ok) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const float4 v = make_float4(oacc[db][4 * ig], oacc[db][4 * ig + 1], oacc[db][4 * ig + 2],
                                       oacc[db][4 * ig + 3]);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), ro,
                                                 obase + (32 * db + 8 * ig) * 4, 0, kCoherent);
        }
      if (hh == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, lse_here), rl, (int)(qrow * 4), 0,
                                              kCoherent);
    }
  }
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __builtin_amdgcn_atomic_inc32(a.counters + (int64_t)pair * a.row_tiles + tile,
                                                       (unsigned)(members - 1), __ATOMIC_RELAXED, "agent");
    s_last = (old == (unsigned)(members - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last || !row_ok) return;
  // Last arrival: combine every member's partial, always in member order, so
  // the result does not depend on which workgroup arrived last. Pass 1 finds
  // the largest lse; pass 2 sums the weighted outputs (independent loads).
  float lmax = neg_inf();
  for (int sp = 0; sp < members; ++sp) {
    const __amdgpu_buffer_rsrc_t rl = coherent_rsrc(a.part_lse + (int64_t)sp * rows, rows);
    lmax = fmaxf(lmax, __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, (int)(qrow * 4), 0, kCoherent)));
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float wsum = 0.f;
  if (lmax != neg_inf()) {
    for (int sp = 0; sp < members; ++sp) {
      const __amdgpu_buffer_rsrc_t ro = coherent_rsrc(a.part_o + (int64_t)sp * rows * D, rows * D);
      const __amdgpu_buffer_rsrc_t rl = coherent_rsrc(a.part_lse + (int64_t)sp * rows, rows);
      const float lo = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, (int)(qrow * 4), 0, kCoherent));
      const float w = exp2_approx((lo - lmax) * kLog2e);  // empty member: exp2(-inf) = 0
      wsum += w;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const float4 v = __builtin_bit_cast(
              float4, __builtin_amdgcn_raw_buffer_load_b128(ro, obase + (32 * db + 8 * ig) * 4, 0, kCoherent));
          if (w != 0.f) {
            oacc[db][4 * ig + 0] += w * v.x;
            oacc[db][4 * ig + 1] += w * v.y;
            oacc[db][4 * ig + 2] += w * v.z;
            oacc[db][4 * ig + 3] += w * v.w;
          }
        }
    }
  }
  const float winv = wsum > 0.f ? 1.0f / wsum : 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] *= winv;
  store_rows<D>(a.out.o + qrow * D + 4 * hh, oacc);
  if (a.out.lse && hh == 0) a.out.lse[qrow] = wsum > 0.f ? lmax + log2_approx(wsum) * kLn2 : neg_inf();
#endif
}

template <int D, int NW>
hipError_t launch_dw(const SharedMfmaArgs& a, int64_t grid, int64_t n_logical, hipStream_t st) {
  if (a.stages == 4)
    hipLaunchKernelGGL((shared_mfma_kernel<D, NW, 4>), dim3((unsigned)grid), dim3(NW * 64), 0, st, a, n_logical);
  else
    hipLaunchKernelGGL((shared_mfma_kernel<D, NW, 2>), dim3((unsigned)grid), dim3(NW * 64), 0, st, a, n_logical);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const SharedMfmaArgs& a, hipStream_t st) {
  const int members = a.p_splits + (a.gen_member ? 1 : 0);
  const int64_t n_logical = (int64_t)a.s.R * a.s.Hkv * members * a.row_tiles;
  if (n_logical == 0) return hipSuccess;
  const int64_t grid = (n_logical + 7) / 8 * 8;
  switch (a.waves) {
    case 1: return launch_dw<D, 1>(a, grid, n_logical, st);
    case 2: return launch_dw<D, 2>(a, grid, n_logical, st);
    default: return launch_dw<D, 4>(a, grid, n_logical, st);
  }
}

}  // namespace

hipError_t launch_shared_mfma(const SharedMfmaArgs& a, hipStream_t st) {
  return a.s.D == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace xattn

// Kernel parameter blocks and host launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

// Where a stage writes: the final outputs, or partial slot `part` of the
// workspace (partials are [parts][N_b*H_q][D] and [parts][N_b*H_q]).
struct OutSpec {
  float* o;
  float* lse;           // may be null for final outputs
  int64_t part_stride;  // rows between partial slots (N_b*H_q); 0 for final
  int part_base;        // first partial slot this launch writes
};

struct Shape {
  int R, B, Hq, Hkv, D, T_max;
  int64_t n_ptok;
  float scale_log2;  // softmax scale * log2(e)
};

// ---- Shared stage, bf16 MFMA (shared_mfma.hip) ----
// kModeFinal: one prompt split, write o/lse. kModePartial: write partial slot
// out.part_base + split. kModeFixup: write partial slot `split`, and the last
// workgroup of each (request, kv head, row tile) merges all splits into o/lse.
constexpr int kModeFinal = 0;
constexpr int kModePartial = 1;
constexpr int kModeFixup = 2;

struct SharedMfmaArgs {
  Shape s;
  const uint16_t* q;
  const uint16_t* k_shared;
  const uint16_t* v_shared;
  const int64_t* prefix_off;
  const int32_t* prefix_len;
  // Non-Shared part folded into the epilogue of prefix split 0 (null = none)
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* slot_table;
  const int32_t* unshared_len;
  OutSpec out;      // final outputs (part_base used in kModePartial)
  int mode;
  float* part_o;    // [parts][N_b*H_q][D] partial outputs (modes partial / fixup)
  float* part_lse;  // [parts][N_b*H_q]
  int64_t part_stride;  // N_b*H_q
  unsigned* counters;   // [R*H_kv*row_tiles], zero between calls (fixup)
  int waves;        // waves per block: 1, 2, 4 or 8 (32 query rows each per key group)
  int row_tiles;
  int p_splits;
  int p_chunk;      // multiple of 64
  int gen_member;   // kModeFixup with k_pool: one extra member per group does the Non-Shared tokens
  int stages;       // LDS pipeline stages: 2 or 4
  int key_groups;   // 1, 2 or 4 wave groups splitting each workgroup's keys
  int stream_kv;    // prompt keys read by this workgroup alone: non-temporal loads
  // Fused cache append (kModeFinal, one member): slot_table is the table
  // read (table_in), the new token of each active beam comes from
  // k_new/v_new, and the launch also writes its pool rows, table_out and
  // the new lengths, counting arrivals on unshared_len like the append.
  int append;               // 0: plain decode
  const uint16_t* k_new;    // [N_b][H_kv][D]
  const uint16_t* v_new;
  const int32_t* parent;    // [N_b]
  const int64_t* slot_base; // [R]
  const uint8_t* active;    // [R] or null
  uint16_t* k_pool_out;     // = k_pool, written
  uint16_t* v_pool_out;
  int32_t* table_out;       // [N_b][T_max], not table_in
  int32_t* ulen_rw;         // = unshared_len, counted and written
  // four key groups may take the generated tokens as one matrix-core block:
  // four query heads per kv head, at most three generated tokens, pool and
  // k_new byte offsets within 32 bits
  int token_block;
  uint32_t pool_bytes;      // with token_block: bytes of k_pool (= of v_pool)
  uint32_t new_bytes;       // with token_block and the fused append: bytes of k_new
  int arrivals;             // kv heads per request: second-level arrivals
  // first-level arrivals: `counters` [R*H_kv], the row tiles of a (request,
  // kv head), wrapping back to zero
};
hipError_t launch_shared_mfma(const SharedMfmaArgs& a, hipStream_t st);

// ---- Vector-ALU attention over prompt and/or generated keys (valu_attn.hip) ----
struct ValuArgs {
  Shape s;
  int dtype;  // 0 f32, 1 bf16 (storage of q and K/V)
  const void* q;
  const void* k_shared;
  const void* v_shared;
  const int64_t* prefix_off;
  const int32_t* prefix_len;
  const void* k_pool;
  const void* v_pool;
  const int32_t* slot_table;
  const int32_t* unshared_len;
  int use_prefix, use_gen;
  int splits;       // key-range splits (over the prompt if use_prefix, else over generated)
  int chunk;        // keys per split
  OutSpec out;      // writes slot part_base + split when out.part_stride != 0
  // Partials folded into the final output by the LSE rule (the prompt
  // splits an earlier launch wrote): fold_parts slots of [fold_stride][D]
  // and [fold_stride]; 0 = none. Needs final outputs, and splits merged in
  // one workgroup (splits <= kValuWgMaxSplits).
  const float* fold_o;
  const float* fold_lse;
  int fold_parts;
  int64_t fold_stride;
};
constexpr int kValuWgMaxSplits = 8;  // splits merged inside one workgroup (one wave each), at most
hipError_t launch_valu_attn(const ValuArgs& a, hipStream_t st);

// ---- Merge (merge.hip) ----
hipError_t launch_merge2(int64_t rows, int D, const float* o_a, const float* lse_a, const float* o_b,
                         const float* lse_b, float* o_out, float* lse_out, hipStream_t st);
// Reduce `parts` partial slots [parts][rows][D] into final o/lse (lse nullable).
hipError_t launch_merge_parts(int64_t rows, int D, int parts, const float* po, const float* plse,
                              float* o, float* lse, hipStream_t st);

// ---- Append (append.hip) ----
struct AppendArgs {
  int R, B, Hkv, D, T_max, elem_bytes;
  const void* k_new;
  const void* v_new;
  const int32_t* parent;
  const int64_t* slot_base;
  const uint8_t* active;
  void* k_pool;
  void* v_pool;
  const int32_t* table_in;
  int32_t* table_out;
  int32_t* unshared_len;
};
// One launch per append; its workgroups count their arrivals in the bits of
// unshared_len[r] from kArrivalShift up, so lengths stay below 2^kArrivalShift
// and a request has at most kMaxAppendBlocks workgroups.
constexpr int kArrivalShift = 20;
constexpr int kMaxAppendBlocks = 2047;
bool append_supported(const AppendArgs& a);
hipError_t launch_append(const AppendArgs& a, hipStream_t st);

// ---- Beam-search survivor selection (topk.hip) ----
constexpr int kTopkCap = 8192;        // candidate keys held in LDS per request
constexpr int kTopkMaxBeams = 8192;   // beams per request
constexpr int kTopkMaxOut = 4096;     // survivors per request
struct TopkArgs {
  int R, BW, K, n_out;
  const float* beam_score;  // [R][BW]
  const float* logprob;     // [R][BW][K], each row descending
  const int32_t* token;     // [R][BW][K]
  int32_t* parent;          // [R][n_out]
  int32_t* token_out;       // [R][n_out]
  float* score_out;         // [R][n_out]
};
hipError_t launch_beam_topk(const TopkArgs& a, hipStream_t st);

// ---- PagedAttention-style baseline (paged_attn.hip) ----
constexpr int kPagedBlock = 16;   // tokens per cache block
constexpr int kPagedPart = 512;   // tokens per partition of one beam's sequence
struct PagedArgs {
  int Hq, Hkv, D, max_blocks, nparts;
  int64_t rows;                   // N_b * H_q
  float scale_log2;
  const uint16_t* q;              // [N_b][H_q][D] bf16
  const uint16_t* k_cache;        // [num_blocks][H_kv][kPagedBlock][D]
  const uint16_t* v_cache;
  const int32_t* block_table;     // [N_b][max_blocks]
  const int32_t* seq_len;         // [N_b]
  float* o;                       // [N_b][H_q][D]
  float* lse;                     // [N_b][H_q] or null
  float* part_o;                  // [nparts][rows][D] when nparts > 1
  float* part_lse;                // [nparts][rows]
};
hipError_t launch_paged_attn(const PagedArgs& a, hipStream_t st);
hipError_t launch_copy_blocks(uint16_t* kc, uint16_t* vc, const int32_t* src, const int32_t* dst, int n,
                              int64_t block_elems, hipStream_t st);

// ---- Streaming-read measurement (stream.hip) ----
hipError_t launch_stream_read(const void* src, int64_t bytes, unsigned* sink, hipStream_t st);

}  // namespace xattn

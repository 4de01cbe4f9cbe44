// Token-granular Non-Shared cache append (xGR page, section 2.1 xAttention:
// token-level management of the Non-Shared cache and in-place updates through
// direct indices without read-before-write hazards).
//
// Slot-table column j of a new beam depends only on column j of its parent's
// row, so the table update splits into independent column chunks. One
// workgroup owns one (request, column chunk): it reads the chunk of every
// parent row of the request into LDS, waits at a barrier, then writes the new
// rows. No other workgroup touches those table cells, so table_out may alias
// table_in. Further workgroups of the same launch copy the new K/V rows into
// their pool slots. A second one-block launch increments unshared_len after
// both have read it.
#include "device.h"
#include "kernels.h"

namespace xattn {

namespace {

constexpr int kAppendThreads = 256;
constexpr int kTableLdsInts = 8192;  // 32 KiB of staged table cells per workgroup

struct AppendPlan {
  int col_chunk;     // table columns per workgroup
  int col_blocks;    // workgroups per request for the table
  int kv_blocks;     // workgroups per request for the K/V copy
};

AppendPlan plan_append(const AppendArgs& a) {
  AppendPlan p;
  p.col_chunk = kTableLdsInts / a.B;
  if (p.col_chunk < 1) p.col_chunk = 1;
  if (p.col_chunk > a.T_max) p.col_chunk = a.T_max;
  p.col_blocks = (a.T_max + p.col_chunk - 1) / p.col_chunk;
  const int64_t bytes = 2LL * a.B * a.Hkv * a.D * a.elem_bytes;
  int64_t kv = (bytes + 65535) / 65536;
  p.kv_blocks = (int)(kv < 1 ? 1 : (kv > 1024 ? 1024 : kv));
  return p;
}

__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a, AppendPlan p) {
  extern __shared__ int32_t staged[];  // [B][col_chunk]
  const int r = blockIdx.x;
  const int y = blockIdx.y;
  if (a.active && !a.active[r]) return;
  const int t = a.unshared_len[r];
  if (t < 0 || t >= a.T_max) return;  // full row: nothing is written
  const int B = a.B;
  const int64_t nbase = (int64_t)r * B;

  if (y < p.col_blocks) {
    const int c0 = y * p.col_chunk;
    const int c1 = min(t, c0 + p.col_chunk);
    const int nc = c1 - c0;
    if (nc > 0) {
      for (int i = threadIdx.x; i < B * nc; i += blockDim.x) {
        const int b = i / nc, c = i - b * nc;
        staged[b * p.col_chunk + c] = a.table_in[(nbase + b) * a.T_max + c0 + c];
      }
      __syncthreads();
      for (int i = threadIdx.x; i < B * nc; i += blockDim.x) {
        const int b = i / nc, c = i - b * nc;
        const int par = a.parent[nbase + b];
        a.table_out[(nbase + b) * a.T_max + c0 + c] = staged[par * p.col_chunk + c];
      }
    }
    if (y == 0) {
      const int64_t sb = a.slot_base[r] + (int64_t)t * B;
      for (int b = threadIdx.x; b < B; b += blockDim.x)
        a.table_out[(nbase + b) * a.T_max + t] = (int32_t)(sb + b);
    }
    return;
  }

  // K/V copy: 16-byte pieces of each beam's [H_kv][D] row.
  const int64_t row_bytes = (int64_t)a.Hkv * a.D * a.elem_bytes;
  const int64_t pieces = row_bytes / 16;
  const int64_t total = pieces * B;
  const int64_t sb = a.slot_base[r] + (int64_t)t * B;
  const int kvb = y - p.col_blocks;
  for (int64_t i = (int64_t)kvb * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)p.kv_blocks * blockDim.x) {
    const int64_t b = i / pieces, k = i - b * pieces;
    const int64_t src = (nbase + b) * row_bytes + k * 16;
    const int64_t dst = (sb + b) * row_bytes + k * 16;
    const uint4 kv = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + src);
    const uint4 vv = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_new) + src);
    *reinterpret_cast<uint4*>(static_cast<char*>(a.k_pool) + dst) = kv;
    *reinterpret_cast<uint4*>(static_cast<char*>(a.v_pool) + dst) = vv;
  }
}

__global__ __launch_bounds__(256) void append_bump_kernel(int R, int T_max, const uint8_t* active,
                                                          int32_t* unshared_len) {
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < R; r += gridDim.x * blockDim.x) {
    if (active && !active[r]) continue;
    const int t = unshared_len[r];
    if (t >= 0 && t < T_max) unshared_len[r] = t + 1;
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  if (a.R == 0) return hipSuccess;
  const AppendPlan p = plan_append(a);
  const size_t lds = (size_t)a.B * p.col_chunk * sizeof(int32_t);
  dim3 grid(a.R, p.col_blocks + p.kv_blocks);
  hipLaunchKernelGGL(append_kernel, grid, dim3(kAppendThreads), lds, st, a, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = (a.R + 255) / 256;
  hipLaunchKernelGGL(append_bump_kernel, dim3(nb), dim3(256), 0, st, a.R, a.T_max, a.active,
                     a.unshared_len);
  return hipGetLastError();
}

}  // namespace xattn

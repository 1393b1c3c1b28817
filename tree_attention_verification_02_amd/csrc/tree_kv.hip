// Tree mask construction, KV append and KV commit/rollback kernels.
//
// Mask: page "投机推理算法的常见优化手段" (cnblogs), tree-mask section -- each
// flattened tree token attends only to its ancestors; the printed matrix has
// row = attending token, column = attended token and a set diagonal.  Here
// each row's mask is packed into 64-bit words (bit j%64 of word j/64 is the
// entry for local row j).
//
// Commit: guijiagi.com speculative-decoding post, KV-cache management section
// -- rejected candidates' KV is rolled back; with paged KV their blocks are
// freed.  The accepted path is compacted to the front of the tree's slots.
#include "common.hpp"
#include "launch.hpp"

namespace spec {

// One workgroup per request, one thread per row (blockDim = kMaxRows).
__global__ void __launch_bounds__(kMaxRows)
build_mask_kernel(const int32_t* __restrict__ row_offsets, const int32_t* __restrict__ prefix_len,
                  const int32_t* __restrict__ parents, uint64_t* __restrict__ mask, int words,
                  int32_t* __restrict__ depth_out, int32_t* __restrict__ pos_out,
                  int32_t* __restrict__ err_row) {
  __shared__ int par[kMaxRows];
  __shared__ int bad;
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int o = row_offsets[b];
  const int n = row_offsets[b + 1] - o;
  if (i == 0) bad = 0x7fffffff;
  if (i < n) par[i] = parents[o + i];
  __syncthreads();
  if (i < n) {
    const int p = par[i];
    const bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i);
    if (!ok) atomicMin(&bad, i);
  }
  __syncthreads();
  if (i >= n) return;
  uint64_t w[kMaxWords] = {0, 0, 0, 0};
  int d = -1;
  if (bad == 0x7fffffff) {
    // parent[j] < j for every row, so the walk strictly descends to the root
    for (int j = i; j >= 0; j = par[j]) {
      w[j >> 6] |= 1ull << (j & 63);
      ++d;
    }
  }
  for (int k = 0; k < words; ++k) mask[(int64_t)(o + i) * words + k] = w[k];
  if (depth_out) depth_out[o + i] = d;
  if (pos_out) pos_out[o + i] = (d < 0) ? -1 : prefix_len[b] + d;
  if (i == 0) err_row[b] = (bad == 0x7fffffff) ? -1 : bad;
}

// Batches up to this many requests keep their row offsets in LDS.
constexpr int kAppendLdsRows = 4096;

// One thread per 16-byte chunk of a new K or V row.
__global__ void __launch_bounds__(256)
kv_append_kernel(const int32_t* __restrict__ row_offsets, const int32_t* __restrict__ prefix_len,
                 int B, int R, KvAddr addr, int esize, const uint4* __restrict__ k_new,
                 const uint4* __restrict__ v_new, char* __restrict__ k_cache,
                 char* __restrict__ v_cache) {
  // the row offsets go to LDS first (one load round trip), so that finding
  // each row's request is a search in LDS rather than a chain of dependent
  // global loads; larger batches search in global memory
  __shared__ int s_ro[kAppendLdsRows + 1];
  const bool in_lds = B <= kAppendLdsRows;
  if (in_lds) {
    for (int i = threadIdx.x; i <= B; i += blockDim.x) s_ro[i] = row_offsets[i];
    __syncthreads();
  }
  const int32_t* ro = in_lds ? s_ro : row_offsets;
  const int chunks = addr.d * esize / 16;           // per (row, head)
  const int64_t total = (int64_t)R * addr.hkv * chunks;
  int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; id < 2 * total; id += stride) {
    const bool is_v = id >= total;
    const int64_t e = is_v ? id - total : id;
    const int c = (int)(e % chunks);
    const int h = (int)((e / chunks) % addr.hkv);
    const int r = (int)(e / ((int64_t)chunks * addr.hkv));
    const int b = request_of_row(ro, B, r);
    const int t = prefix_len[b] + (r - ro[b]);
    const int64_t dst = addr(b, h, t) * esize + (int64_t)c * 16;
    const uint4 val = is_v ? v_new[e] : k_new[e];
    *reinterpret_cast<uint4*>((is_v ? v_cache : k_cache) + dst) = val;
  }
}

// One workgroup per (request, KV head).  Rows are moved in blocks of
// `kCommitRows`: all reads of a block finish (barrier) before its writes.
// Because path[k] >= k, a write to slot L+k can only clobber the source of an
// earlier k' (already read), never of a later one, so blocked in-order
// copying is safe in place.
constexpr int kCommitRows = 16;

__global__ void __launch_bounds__(256)
kv_commit_kernel(const int32_t* __restrict__ row_offsets, const int32_t* __restrict__ prefix_len,
                 KvAddr addr, int esize, const int32_t* __restrict__ accept_len,
                 const int32_t* __restrict__ path, int path_stride, char* __restrict__ k_cache,
                 char* __restrict__ v_cache, int32_t* __restrict__ new_len,
                 int32_t* __restrict__ freed) {
  static_assert(kMaxRows <= 256, "one thread per path entry");
  const int b = blockIdx.x / addr.hkv;
  const int h = blockIdx.x % addr.hkv;
  const int tid = threadIdx.x;
  __shared__ int pth[kMaxRows];
  // one memory round trip: the request's bounds, accept_len and its path row
  const int o = row_offsets[b];
  const int n = row_offsets[b + 1] - o;
  const int L = prefix_len[b];
  const int a = accept_len[b];
  const int lim = min(path_stride, kMaxRows);
  const int pk = (tid < lim) ? path[(int64_t)b * path_stride + tid] : -1;
  if (tid < lim) pth[tid] = pk;
  __syncthreads();
  // the path must start at the root and increase strictly within the tree
  const bool a_ok = a >= 0 && a < n && a < path_stride;
  bool bad = !a_ok;
  if (a_ok && tid <= a) bad = (tid == 0) ? (pk != 0) : !(pk > pth[tid - 1] && pk < n);
  if (__syncthreads_or(bad)) {
    if (h == 0 && tid == 0) new_len[b] = -1;
    return;
  }
  const int nl = L + a + 1;
  if (h == 0) {
    if (tid == 0) new_len[b] = nl;
    if (freed && addr.paged) {
      const int first = (nl + kBlock - 1) / kBlock;
      const int end = (L + n + kBlock - 1) / kBlock;
      for (int j = tid; j < addr.mbps; j += blockDim.x) {
        const int src = first + j;
        freed[(int64_t)b * addr.mbps + j] =
            (src < end) ? addr.block_table[(int64_t)b * addr.mbps + src] : -1;
      }
    }
  }
  // rows already in place (path[k] == k, e.g. an accepted first child) are
  // neither read nor written
  if (!__syncthreads_or(tid >= 1 && tid <= a && pk != tid)) return;
  const int chunks = addr.d * esize / 16;
  for (int k0 = 1; k0 <= a; k0 += kCommitRows) {
    const int rows = min(kCommitRows, a + 1 - k0);
    const int items = rows * chunks * 2;            // K and V
    // items <= kCommitRows * 32 chunks * 2 = 1024 = 4 per thread
    uint4 buf[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int it = tid + q * 256;
      if (it < items) {
        const int isv = it / (rows * chunks);
        const int rem = it % (rows * chunks);
        const int k = k0 + rem / chunks;
        const int c = rem % chunks;
        if (pth[k] != k) {
          const int64_t src = addr(b, h, L + pth[k]) * esize + (int64_t)c * 16;
          buf[q] = *reinterpret_cast<const uint4*>((isv ? v_cache : k_cache) + src);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int it = tid + q * 256;
      if (it < items) {
        const int isv = it / (rows * chunks);
        const int rem = it % (rows * chunks);
        const int k = k0 + rem / chunks;
        const int c = rem % chunks;
        if (pth[k] != k) {
          const int64_t dst = addr(b, h, L + k) * esize + (int64_t)c * 16;
          *reinterpret_cast<uint4*>((isv ? v_cache : k_cache) + dst) = buf[q];
        }
      }
    }
    __syncthreads();
  }
}

hipError_t launch_build_mask(const LaunchCtx& cx, const int32_t* parents, uint64_t* mask, int words,
                             int32_t* depth, int32_t* pos, int32_t* err_row) {
  hipLaunchKernelGGL(build_mask_kernel, dim3(cx.B), dim3(kMaxRows), 0, cx.stream,
                     cx.row_offsets_d, cx.prefix_len_d, parents, mask, words, depth, pos, err_row);
  return hipGetLastError();
}

hipError_t launch_kv_append(const LaunchCtx& cx, int R, const KvAddr& addr, int esize,
                            const void* k_new, const void* v_new, void* k_cache, void* v_cache) {
  const int64_t total = 2ll * R * addr.hkv * (addr.d * esize / 16);
  int grid = (int)((total + 255) / 256);
  if (grid > 65536) grid = 65536;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kv_append_kernel, dim3(grid), dim3(256), 0, cx.stream, cx.row_offsets_d,
                     cx.prefix_len_d, cx.B, R, addr, esize, (const uint4*)k_new,
                     (const uint4*)v_new, (char*)k_cache, (char*)v_cache);
  return hipGetLastError();
}

hipError_t launch_kv_commit(const LaunchCtx& cx, const KvAddr& addr, int esize,
                            const int32_t* accept_len, const int32_t* path, int path_stride,
                            void* k_cache, void* v_cache, int32_t* new_len, int32_t* freed) {
  hipLaunchKernelGGL(kv_commit_kernel, dim3(cx.B * addr.hkv), dim3(256), 0, cx.stream,
                     cx.row_offsets_d, cx.prefix_len_d, addr, esize, accept_len, path,
                     path_stride, (char*)k_cache, (char*)v_cache, new_len, freed);
  return hipGetLastError();
}

}  // namespace spec

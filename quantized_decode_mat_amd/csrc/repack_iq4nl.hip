// repack_iq4nl.hip — IQ4_NL file blocks -> resident rows, once, at upload.
//
// "25 — Writing XPU Kernels", section 25.4: weights are converted once when
// they are bound, into the one resident layout every kernel reads (a row is
// its f16 block scales padded to a dword, then its 16-byte payloads), and the
// copy is mapped like the decode kernels: each work item moves one dword of
// payload rather than a wave taking a whole block. A separate pass over the
// scattered scale bytes would pull a cache line per block for two useful
// bytes, so the scale goes with the pass that already reads those lines
// (section 25.4.1 leaves that fold open).
//
// Source: a chunk of the file's 18-byte blocks (f16 scale at +0, then the 16
// payload bytes), global blocks block_base .. block_base + n - 1 of a matrix
// of bpr blocks per row. The source is 2-byte aligned at best (18-byte
// stride), so it is read as 16-bit halves; every resident store is a dword or
// a 16-bit half at its natural alignment.
//
// Two routes, both one pass:
//  * any chunk: work item t writes payload dword t%4 of block t/4; the item
//    with t%4 == 0 also writes the block's scale as a 16-bit store, and, for
//    the last block of a row with an odd bpr, the zero pad half after it;
//  * a chunk that starts and ends on row boundaries: the payload items as
//    above, plus one item per prefix dword writing two scales (or a scale and
//    the zero pad) at once, so every resident store is a full dword. The host
//    counts launches of this route so a test can see that it fires.
#include <atomic>

#include "xq_device.h"
#include "xq_launch.h"

namespace xq {
namespace {

constexpr int kRepackThreads = 256;
constexpr int kFileBlockBytes = 18;

__device__ __forceinline__ uint32_t src_half(const uint16_t* src, int64_t byte_off) {
  return src[byte_off >> 1];
}

// I: the type of the block and item indices. 32-bit when every index of the
// chunk fits (the host checks): a 64-bit division by bpr is a long software
// sequence per work item, a 32-bit one a few instructions. Byte offsets stay
// 64-bit either way.
template <bool DWORD_PREFIX, typename I>
__global__ __launch_bounds__(kRepackThreads) void repack_iq4nl_kernel(
    uint8_t* __restrict__ out, const uint16_t* __restrict__ src, int64_t n64, int64_t base64,
    int64_t bpr64, int64_t prefix, int64_t row_bytes, int64_t prefix_items64) {
  const I n = static_cast<I>(n64);
  const I block_base = static_cast<I>(base64);
  const I bpr = static_cast<I>(bpr64);
  const I prefix_items = static_cast<I>(prefix_items64);
  const I t = static_cast<I>(blockIdx.x) * kRepackThreads + static_cast<I>(threadIdx.x);
  const I pay_items = 4 * n;
  if (t < pay_items) {
    const I b = t >> 2;  // block within the chunk
    const int k = static_cast<int>(t & 3);
    const I gb = block_base + b;
    const I row = gb / bpr;
    const I j = gb - row * bpr;
    const int64_t so = static_cast<int64_t>(b) * kFileBlockBytes + 2 + 4 * k;
    const uint32_t w = src_half(src, so) | (src_half(src, so + 2) << 16);
    uint8_t* orow = out + static_cast<int64_t>(row) * row_bytes;
    *reinterpret_cast<uint32_t*>(orow + prefix + 16 * static_cast<int64_t>(j) + 4 * k) = w;
    if (!DWORD_PREFIX && k == 0) {
      reinterpret_cast<uint16_t*>(orow)[j] =
          static_cast<uint16_t>(src_half(src, static_cast<int64_t>(b) * kFileBlockBytes));
      if (j == bpr - 1 && (bpr & 1)) reinterpret_cast<uint16_t*>(orow)[j + 1] = 0;
    }
    return;
  }
  if (DWORD_PREFIX) {
    const I p = t - pay_items;  // prefix dword over the chunk's rows
    if (p >= prefix_items) return;
    const I pw = static_cast<I>(prefix >> 2);
    const I r = p / pw;                 // row within the chunk
    const I i = p - r * pw;             // dword within the prefix
    const I b0 = r * bpr + 2 * i;       // block within the chunk
    const uint32_t lo = src_half(src, static_cast<int64_t>(b0) * kFileBlockBytes);
    const uint32_t hi =
        (2 * i + 1 < bpr) ? src_half(src, static_cast<int64_t>(b0 + 1) * kFileBlockBytes) : 0u;
    const int64_t row = static_cast<int64_t>(block_base / bpr) + r;
    *reinterpret_cast<uint32_t*>(out + row * row_bytes + 4 * static_cast<int64_t>(i)) =
        lo | (hi << 16);
  }
}

// The tiled form, for a 16-byte aligned source: a workgroup stages 256 file
// blocks (4608 bytes, a whole number of 16-byte chunks) into LDS with 16-byte
// loads, then each item moves one whole block from LDS: its 16 payload bytes
// as one 16-byte store where the destination is 16-byte aligned (four dword
// stores otherwise), and its scale. The 2-byte loads of the direct form bring
// a wave 128 bytes per load instruction; the staging brings 1 KiB, and one
// row division per block replaces four. Both routes as above: the scale goes
// as a half (and the pad after an odd row's last scale), or, in the
// dword-prefix route when the block starts a scale pair (even index within
// its row), as the pair's dword; the pair's second scale comes from the tile,
// or from global memory when the pair straddles the tile's end.
constexpr int kTileBlocks = 256;
constexpr int kTileBytes = kTileBlocks * kFileBlockBytes;
static_assert(kTileBytes % 16 == 0, "a tile is whole 16-byte chunks");

template <bool DWORD_PREFIX, typename I>
__global__ __launch_bounds__(kRepackThreads) void repack_iq4nl_tiled_kernel(
    uint8_t* __restrict__ out, const uint8_t* __restrict__ src, int64_t n64, int64_t base64,
    int64_t bpr64, int64_t prefix, int64_t row_bytes) {
  __shared__ __align__(16) uint16_t tile[kTileBytes / 2];
  const I n = static_cast<I>(n64);
  const I block_base = static_cast<I>(base64);
  const I bpr = static_cast<I>(bpr64);
  const I b0 = static_cast<I>(blockIdx.x) * kTileBlocks;  // the tile's first block in the chunk
  const int nb = static_cast<int>(min(n - b0, static_cast<I>(kTileBlocks)));
  const uint8_t* tsrc = src + static_cast<int64_t>(b0) * kFileBlockBytes;
  const int bytes = nb * kFileBlockBytes;  // even
  const int full = bytes >> 4;             // whole 16-byte chunks inside the chunk
  for (int c = threadIdx.x; c < full; c += kRepackThreads)
    reinterpret_cast<uint4*>(tile)[c] = reinterpret_cast<const uint4*>(tsrc)[c];
  for (int h = 8 * full + threadIdx.x; h < (bytes >> 1); h += kRepackThreads)
    tile[h] = reinterpret_cast<const uint16_t*>(tsrc)[h];
  __syncthreads();

  for (int b = threadIdx.x; b < nb; b += kRepackThreads) {
    const I gb = block_base + b0 + static_cast<I>(b);
    const I row = gb / bpr;
    const I j = gb - row * bpr;
    const int hb = (b * kFileBlockBytes) >> 1;  // the block's first half in the tile
    uint4 p;
    p.x = static_cast<uint32_t>(tile[hb + 1]) | (static_cast<uint32_t>(tile[hb + 2]) << 16);
    p.y = static_cast<uint32_t>(tile[hb + 3]) | (static_cast<uint32_t>(tile[hb + 4]) << 16);
    p.z = static_cast<uint32_t>(tile[hb + 5]) | (static_cast<uint32_t>(tile[hb + 6]) << 16);
    p.w = static_cast<uint32_t>(tile[hb + 7]) | (static_cast<uint32_t>(tile[hb + 8]) << 16);
    uint8_t* orow = out + static_cast<int64_t>(row) * row_bytes;
    uint8_t* dst = orow + prefix + 16 * static_cast<int64_t>(j);
    if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      *reinterpret_cast<uint4*>(dst) = p;
    } else {
      uint32_t* d4 = reinterpret_cast<uint32_t*>(dst);
      d4[0] = p.x; d4[1] = p.y; d4[2] = p.z; d4[3] = p.w;
    }
    const uint32_t sc = tile[hb];
    if (!DWORD_PREFIX) {
      reinterpret_cast<uint16_t*>(orow)[j] = static_cast<uint16_t>(sc);
      if (j == bpr - 1 && (bpr & 1)) reinterpret_cast<uint16_t*>(orow)[j + 1] = 0;
    } else if ((j & 1) == 0) {
      uint32_t hi = 0;
      if (j + 1 < bpr)
        hi = (b + 1 < nb) ? tile[((b + 1) * kFileBlockBytes) >> 1]
                          : reinterpret_cast<const uint16_t*>(tsrc)[((b + 1) * kFileBlockBytes) >> 1];
      *reinterpret_cast<uint32_t*>(orow + 2 * static_cast<int64_t>(j)) = sc | (hi << 16);
    }
  }
}

std::atomic<int64_t> g_dword_prefix_launches{0};

}  // namespace

int64_t repack_dword_prefix_launches() {
  return g_dword_prefix_launches.load(std::memory_order_relaxed);
}

hipError_t launch_repack_iq4nl(void* resident, const void* file_blocks, int64_t n,
                               int64_t block_base, int64_t bpr, hipStream_t stream) {
  const int64_t prefix = ((2 * bpr + 3) / 4) * 4;
  const int64_t row_bytes = prefix + 16 * bpr;
  const bool row_aligned = (block_base % bpr == 0) && (n % bpr == 0);
  const int64_t prefix_items = row_aligned ? (n / bpr) * (prefix / 4) : 0;
  const int64_t items = 4 * n + prefix_items;
  const int64_t grid = (items + kRepackThreads - 1) / kRepackThreads;
  uint8_t* out = static_cast<uint8_t*>(resident);
  const uint16_t* src = static_cast<const uint16_t*>(file_blocks);
  if ((reinterpret_cast<uintptr_t>(file_blocks) & 15) == 0) {
    // The tiled form (16-byte aligned source). Its indices: block and row
    // indices below block_base + n, tile indices below n / 256.
    const int64_t tiles = (n + kTileBlocks - 1) / kTileBlocks;
    const bool t32 = block_base + n < (int64_t{1} << 32);
    const uint8_t* s8 = static_cast<const uint8_t*>(file_blocks);
    if (row_aligned) {
      if (t32)
        hipLaunchKernelGGL((repack_iq4nl_tiled_kernel<true, uint32_t>),
                           dim3(static_cast<uint32_t>(tiles)), dim3(kRepackThreads), 0, stream, out,
                           s8, n, block_base, bpr, prefix, row_bytes);
      else
        hipLaunchKernelGGL((repack_iq4nl_tiled_kernel<true, int64_t>),
                           dim3(static_cast<uint32_t>(tiles)), dim3(kRepackThreads), 0, stream, out,
                           s8, n, block_base, bpr, prefix, row_bytes);
      const hipError_t e = hipGetLastError();
      if (e == hipSuccess) g_dword_prefix_launches.fetch_add(1, std::memory_order_relaxed);
      return e;
    }
    if (t32)
      hipLaunchKernelGGL((repack_iq4nl_tiled_kernel<false, uint32_t>),
                         dim3(static_cast<uint32_t>(tiles)), dim3(kRepackThreads), 0, stream, out,
                         s8, n, block_base, bpr, prefix, row_bytes);
    else
      hipLaunchKernelGGL((repack_iq4nl_tiled_kernel<false, int64_t>),
                         dim3(static_cast<uint32_t>(tiles)), dim3(kRepackThreads), 0, stream, out,
                         s8, n, block_base, bpr, prefix, row_bytes);
    return hipGetLastError();
  }
  // 32-bit indices when the largest of them (the grid's items, the last
  // global block) fits below 2^32.
  const int64_t kI32 = int64_t{1} << 32;
  const bool idx32 = grid * kRepackThreads < kI32 && block_base + n < kI32;
  if (row_aligned) {
    if (idx32)
      hipLaunchKernelGGL((repack_iq4nl_kernel<true, uint32_t>), dim3(static_cast<uint32_t>(grid)),
                         dim3(kRepackThreads), 0, stream, out, src, n, block_base, bpr, prefix,
                         row_bytes, prefix_items);
    else
      hipLaunchKernelGGL((repack_iq4nl_kernel<true, int64_t>), dim3(static_cast<uint32_t>(grid)),
                         dim3(kRepackThreads), 0, stream, out, src, n, block_base, bpr, prefix,
                         row_bytes, prefix_items);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) g_dword_prefix_launches.fetch_add(1, std::memory_order_relaxed);
    return e;
  }
  if (idx32)
    hipLaunchKernelGGL((repack_iq4nl_kernel<false, uint32_t>), dim3(static_cast<uint32_t>(grid)),
                       dim3(kRepackThreads), 0, stream, out, src, n, block_base, bpr, prefix,
                       row_bytes, prefix_items);
  else
    hipLaunchKernelGGL((repack_iq4nl_kernel<false, int64_t>), dim3(static_cast<uint32_t>(grid)),
                       dim3(kRepackThreads), 0, stream, out, src, n, block_base, bpr, prefix,
                       row_bytes, prefix_items);
  return hipGetLastError();
}

}  // namespace xq

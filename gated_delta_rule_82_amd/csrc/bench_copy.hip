// bench_copy.hip - streaming copy kernels that give the benchmark its
// practical HBM ceiling: a plain device copy over the same byte count as the
// measured kernel moves (read once, written once).  Built into its own
// library, libkda_bench.so, which only the benchmark loads; nothing of the
// KDA path lives here.
//
// Variants (all move 16-byte pieces through a raw buffer resource spanning
// one workgroup's chunk, so the hardware range check clips a ragged tail):
//   KDA_COPY_STREAM_NT   256 threads per workgroup, 4 pieces per thread,
//                        16 KiB chunks, every access with the nontemporal
//                        cache policy.
//   KDA_COPY_WAVE_NT     one wave per workgroup, 16 pieces per lane
//                        (16 KiB chunks, all loads issued before the first
//                        store, as a decode wave moves its state slab),
//                        nontemporal.
//   KDA_COPY_WAVE        the same with ordinary cached accesses.
//   KDA_COPY_SLAB_NT     the key-first decode's own access pattern: one wave
//                        per 128-byte column slab of a 64 KiB tile of 512-byte
//                        rows (lane (r, c) moves row r + 8 i, bytes 16 c of
//                        the slab), four waves per tile, nontemporal.
// Workgroup ids are remapped so that each of the 8 XCDs walks one contiguous
// range of chunks (consecutive ids land on different XCDs).

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kWave = 64;
constexpr int kXcds = 8;
constexpr int kPolicyNT = 2;
constexpr int kRawBufferWord3 = 0x00020000;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

enum { KDA_COPY_STREAM_NT = 0, KDA_COPY_WAVE_NT = 1, KDA_COPY_WAVE = 2, KDA_COPY_SLAB_NT = 3 };

__device__ __forceinline__ uint32_t xcd_block() {
  const uint32_t wg = blockIdx.x, nwg = gridDim.x;
  const uint32_t xcd = wg % kXcds, per = nwg / kXcds, extra = nwg % kXcds;
  return xcd * per + (xcd < extra ? xcd : extra) + wg / kXcds;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t resource(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           kRawBufferWord3);
}

// Contiguous chunks of THREADS * U * 16 bytes: thread i moves pieces
// i + THREADS * u.
template <int THREADS, int U, int POLICY>
__global__ __launch_bounds__(THREADS) void copy_chunks(char* dst, const char* src, int64_t nbytes) {
  constexpr int kChunk = THREADS * U * 16;
  const int64_t off = static_cast<int64_t>(xcd_block()) * kChunk;
  const int64_t left = nbytes - off;
  const int bytes = left < kChunk ? static_cast<int>(left) : kChunk;
  const __amdgpu_buffer_rsrc_t rs = resource(src + off, bytes);
  const __amdgpu_buffer_rsrc_t rd = resource(dst + off, bytes);
  const int v = static_cast<int>(threadIdx.x) * 16;
  u32x4 x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) x[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, v, u * THREADS * 16, POLICY);
#pragma unroll
  for (int u = 0; u < U; ++u) __builtin_amdgcn_raw_buffer_store_b128(x[u], rd, v, u * THREADS * 16, POLICY);
}

// 64 KiB tiles of 128 rows x 512 bytes; workgroup (tile, slab) moves bytes
// [128 slab, 128 slab + 128) of every row: lane (r = lane / 8, c = lane % 8)
// takes rows r + 8 i, i = 0..15.
constexpr int kTileBytes = 65536;
constexpr int kRowBytes = 512;

__global__ __launch_bounds__(kWave) void copy_slabs(char* dst, const char* src, int64_t nbytes) {
  const uint32_t logical = xcd_block();
  const int slab = static_cast<int>(logical % 4);
  const int64_t off = static_cast<int64_t>(logical / 4) * kTileBytes;
  if (off >= nbytes) return;
  const __amdgpu_buffer_rsrc_t rs = resource(src + off, kTileBytes);
  const __amdgpu_buffer_rsrc_t rd = resource(dst + off, kTileBytes);
  const int lane = static_cast<int>(threadIdx.x);
  const int v = (lane / 8) * kRowBytes + slab * 128 + (lane % 8) * 16;
  u32x4 x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, v, i * 8 * kRowBytes, kPolicyNT);
#pragma unroll
  for (int i = 0; i < 16; ++i) __builtin_amdgcn_raw_buffer_store_b128(x[i], rd, v, i * 8 * kRowBytes, kPolicyNT);
}

}  // namespace

extern "C" {

// Copies nbytes from src to dst (device pointers, 16-byte aligned, nbytes a
// multiple of 16; KDA_COPY_SLAB_NT needs a multiple of 64 KiB) on `stream`.
// Returns 0, -1 for bad arguments, -6 when the launch fails.
int kda_bench_copy(void* dst, const void* src, int64_t nbytes, int variant, hipStream_t stream) {
  if (dst == nullptr || src == nullptr || nbytes <= 0 || nbytes % 16 != 0) return -1;
  if (reinterpret_cast<uintptr_t>(dst) % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0) return -1;
  const void* fn = nullptr;
  int64_t chunk = 0;
  int threads = kWave;
  switch (variant) {
    case KDA_COPY_STREAM_NT:
      fn = reinterpret_cast<const void*>(&copy_chunks<256, 4, kPolicyNT>);
      chunk = 256 * 4 * 16;
      threads = 256;
      break;
    case KDA_COPY_WAVE_NT:
      fn = reinterpret_cast<const void*>(&copy_chunks<kWave, 16, kPolicyNT>);
      chunk = kWave * 16 * 16;
      break;
    case KDA_COPY_WAVE:
      fn = reinterpret_cast<const void*>(&copy_chunks<kWave, 16, 0>);
      chunk = kWave * 16 * 16;
      break;
    case KDA_COPY_SLAB_NT:
      if (nbytes % kTileBytes != 0) return -1;
      fn = reinterpret_cast<const void*>(&copy_slabs);
      chunk = kTileBytes / 4;
      break;
    default:
      return -1;
  }
  const int64_t blocks = (nbytes + chunk - 1) / chunk;
  if (blocks > 0x7fffffff) return -1;
  char* d = static_cast<char*>(dst);
  const char* s = static_cast<const char*>(src);
  void* kargs[] = {&d, &s, &nbytes};
  const hipError_t rc = hipLaunchKernel(fn, dim3(static_cast<uint32_t>(blocks)), dim3(threads), kargs, 0, stream);
  return rc == hipSuccess ? 0 : -6;
}

}  // extern "C"

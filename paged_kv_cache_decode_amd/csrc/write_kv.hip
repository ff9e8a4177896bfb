// Append new tokens' K/V rows into their pool slots (gfx950).
//
// The pool fills block by block, left to right; the caller's allocator
// picks each new token's slot ("Flash Attention vs Paged Attention",
// memory-management paragraph: blocks fill left to right, unfilled slots
// are reserved).  This kernel only moves bytes: one thread copies one
// 16-byte piece of a K row and the same piece of the V row.
#include "device_common.h"
#include "kernels.h"
#include "launch.h"

namespace pa {
namespace {

struct WriteKvArgs {
  const uint8_t* kn;
  const uint8_t* vn;
  int64_t kn_s, kn_h, vn_s, vn_h;  // bytes
  const int32_t* slots;
  uint8_t* kp;
  uint8_t* vp;
  int64_t N;
  int Hkv, row_bytes, chunks;  // chunks = row_bytes / 16
  int B;
  int64_t blk_bytes, tok_bytes, head_bytes;  // pool layout
};

__global__ __launch_bounds__(256) void write_kv_kernel(WriteKvArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_tok = (int64_t)a.Hkv * a.chunks;
  if (idx >= a.N * per_tok) return;
  const int64_t i = idx / per_tok;
  const int rem = (int)(idx % per_tok);
  const int h = rem / a.chunks, ch = rem % a.chunks;
  const int32_t slot = a.slots[i];
  if (slot < 0) return;
  // Slot x is block x / B, position x % B.
  const int64_t dst = (int64_t)(slot / a.B) * a.blk_bytes + (int64_t)(slot % a.B) * a.tok_bytes +
                      h * a.head_bytes + ch * 16;
  *reinterpret_cast<u32x4_t*>(a.kp + dst) = load16(a.kn + i * a.kn_s + h * a.kn_h + ch * 16);
  *reinterpret_cast<u32x4_t*>(a.vp + dst) = load16(a.vn + i * a.vn_s + h * a.vn_h + ch * 16);
}

}  // namespace

hipError_t launch_write_kv(const WriteKvPlan& pl, hipStream_t stream) {
  const int e = pl.dtype == PA_F32 ? 4 : 2;
  WriteKvArgs a;
  a.kn = static_cast<const uint8_t*>(pl.kn);
  a.vn = static_cast<const uint8_t*>(pl.vn);
  a.kn_s = pl.kn_s * e;
  a.kn_h = pl.kn_h * e;
  a.vn_s = pl.vn_s * e;
  a.vn_h = pl.vn_h * e;
  a.slots = pl.slots;
  a.kp = static_cast<uint8_t*>(pl.kp);
  a.vp = static_cast<uint8_t*>(pl.vp);
  a.N = pl.N;
  a.Hkv = pl.Hkv;
  a.row_bytes = pl.D * e;
  a.chunks = a.row_bytes / 16;
  a.B = pl.B;
  a.blk_bytes = (int64_t)pl.B * pl.Hkv * pl.D * e;
  a.tok_bytes = pl.pool.tok * e;
  a.head_bytes = pl.pool.head * e;
  const int64_t total = pl.N * pl.Hkv * a.chunks;
  if (total == 0) return hipSuccess;
  return timed_launch("write_kv", write_kv_kernel, dim3((unsigned)((total + 255) / 256)),
                      dim3(256), stream, a);
}

namespace {

struct CopyBlocksArgs {
  const int32_t* src;
  const int32_t* dst;
  uint8_t* kp;
  uint8_t* vp;
  int64_t chunks;  // 16-byte pieces per block
  int64_t total;   // pairs * chunks
};

// Copy-on-write: whole physical blocks src[i] -> dst[i] in both pools, one
// thread per 16-byte piece of K and the same piece of V.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.total) return;
  const int64_t i = idx / a.chunks, c = idx % a.chunks;
  const int64_t bytes = a.chunks * 16;
  const int64_t from = (int64_t)a.src[i] * bytes + c * 16, to = (int64_t)a.dst[i] * bytes + c * 16;
  *reinterpret_cast<u32x4_t*>(a.kp + to) = load16(a.kp + from);
  *reinterpret_cast<u32x4_t*>(a.vp + to) = load16(a.vp + from);
}

// Shader-clock probe: one wave reads the shader clock counter (s_memtime)
// and the 100 MHz reference counter (s_memrealtime) at its start and once
// `ticks` reference ticks have passed (the loop ends on elapsed real time,
// whatever else the chip is doing), and stores both deltas.
__global__ __launch_bounds__(64) void clock_probe_kernel(int64_t ticks, int64_t* out) {
  const int64_t r0 = (int64_t)__builtin_amdgcn_s_memrealtime();
  const int64_t c0 = (int64_t)__builtin_amdgcn_s_memtime();
  int64_t r = r0;
  while (r - r0 < ticks) {
    __builtin_amdgcn_s_sleep(2);
    r = (int64_t)__builtin_amdgcn_s_memrealtime();
  }
  const int64_t c1 = (int64_t)__builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r - r0;
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksPlan& pl, hipStream_t stream) {
  CopyBlocksArgs a;
  a.src = pl.src;
  a.dst = pl.dst;
  a.kp = static_cast<uint8_t*>(pl.kp);
  a.vp = static_cast<uint8_t*>(pl.vp);
  a.chunks = pl.block_bytes / 16;
  a.total = pl.N * a.chunks;
  if (a.total == 0) return hipSuccess;
  return timed_launch("copy_blocks", copy_blocks_kernel, dim3((unsigned)((a.total + 255) / 256)),
                      dim3(256), stream, a);
}

hipError_t launch_clock_probe(int64_t ticks, int64_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, stream, ticks, out);
  return hipGetLastError();
}

}  // namespace pa

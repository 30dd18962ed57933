// compress_kv: softmax-weighted pooling of m consecutive raw K=V rows into one entry
// (compress_common.h holds the arithmetic and the thread layout). The whole kernel is an HBM
// stream over the raw rows.
#include "compress_common.h"
#include "device_common.h"
#include "launch.h"

namespace csl {

namespace {

template <int TPE, int RS, int RSX, bool HAS_Z, bool OUT_BF16>
__global__ __launch_bounds__(256) void compress_kernel(
    const uint16_t* __restrict__ kv, const uint16_t* __restrict__ z,
    const int64_t* __restrict__ kv_off, const int64_t* __restrict__ ent_off,
    const int64_t* __restrict__ first_entry, int D, int m, int64_t max_new, void* __restrict__ out) {
  // long chunks split over waves hold 8 rows in flight per thread
  compress_block<256, TPE, RS, HAS_Z, OUT_BF16, (RSX > 1 ? 8 : 4), RSX>(kv, z, kv_off, ent_off, first_entry, D, m,
                                                                        max_new, out, blockIdx.y, blockIdx.x);
}

template <int TPE, int RS, int RSX = 1>
hipError_t launch_tpe_rs(const void* kv, const void* z, const int64_t* kv_off, const int64_t* ent_off,
                         const int64_t* first, int B, int D, int m, int64_t max_new, void* out,
                         bool out_bf16, hipStream_t st) {
  constexpr int EPB = 256 / (TPE * RS * RSX);
  const int64_t gx = (max_new + EPB - 1) / EPB;
  dim3 grid((unsigned)gx, (unsigned)B);
  const uint16_t* k16 = static_cast<const uint16_t*>(kv);
  const uint16_t* z16 = static_cast<const uint16_t*>(z);
  if (z) {
    if (out_bf16)
      compress_kernel<TPE, RS, RSX, true, true><<<grid, 256, 0, st>>>(k16, z16, kv_off, ent_off, first, D, m, max_new, out);
    else
      compress_kernel<TPE, RS, RSX, true, false><<<grid, 256, 0, st>>>(k16, z16, kv_off, ent_off, first, D, m, max_new, out);
  } else {
    if (out_bf16)
      compress_kernel<TPE, RS, RSX, false, true><<<grid, 256, 0, st>>>(k16, z16, kv_off, ent_off, first, D, m, max_new, out);
    else
      compress_kernel<TPE, RS, RSX, false, false><<<grid, 256, 0, st>>>(k16, z16, kv_off, ent_off, first, D, m, max_new, out);
  }
  return hipGetLastError();
}

template <int TPE>
hipError_t launch_tpe(const void* kv, const void* z, const int64_t* kv_off, const int64_t* ent_off,
                      const int64_t* first, int B, int D, int m, int64_t max_new, void* out,
                      bool out_bf16, hipStream_t st) {
  constexpr int RS_BIG = (64 / TPE) > 8 ? 8 : (64 / TPE);
  // Few entries (a decode step's newest chunks) of at least 8 rows per in-wave split, with a
  // full wave per entry: split the rows over up to 4 waves too, so a long chunk (m = 128)
  // loads in one round trip. Many entries (bulk compression) keep one wave per entry walking
  // its rows, which streams without workgroup turnover.
  const bool few = (int64_t)B * max_new <= 2048;
  if (few && TPE * RS_BIG == kWave && m >= 8 * RS_BIG * 4)
    return launch_tpe_rs<TPE, RS_BIG, 4>(kv, z, kv_off, ent_off, first, B, D, m, max_new, out, out_bf16, st);
  if (few && TPE * RS_BIG == kWave && m >= 8 * RS_BIG * 2)
    return launch_tpe_rs<TPE, RS_BIG, 2>(kv, z, kv_off, ent_off, first, B, D, m, max_new, out, out_bf16, st);
  if (m > 8 && RS_BIG > 1)
    return launch_tpe_rs<TPE, RS_BIG>(kv, z, kv_off, ent_off, first, B, D, m, max_new, out, out_bf16, st);
  return launch_tpe_rs<TPE, 1>(kv, z, kv_off, ent_off, first, B, D, m, max_new, out, out_bf16, st);
}

}  // namespace

hipError_t launch_compress(const void* kv, const void* z, const int64_t* kv_off, const int64_t* ent_off,
                           const int64_t* first_entry, int B, int D, int m, int64_t max_new_entries,
                           void* out, bool out_bf16, hipStream_t stream) {
  switch (D) {
    case 64: return launch_tpe<8>(kv, z, kv_off, ent_off, first_entry, B, D, m, max_new_entries, out, out_bf16, stream);
    case 128: return launch_tpe<16>(kv, z, kv_off, ent_off, first_entry, B, D, m, max_new_entries, out, out_bf16, stream);
    case 256: return launch_tpe<32>(kv, z, kv_off, ent_off, first_entry, B, D, m, max_new_entries, out, out_bf16, stream);
    case 512: return launch_tpe<64>(kv, z, kv_off, ent_off, first_entry, B, D, m, max_new_entries, out, out_bf16, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace csl

// compress_kv and compress_kv_overlap: softmax-weighted pooling of m consecutive raw K=V rows
// (or, for CSA's overlapped series, of the m rows of series a with the m rows of series b
// before them) into one entry (compress_common.h holds the arithmetic and the thread layout). The whole kernel is an HBM
// stream over the raw rows.
#include "compress_common.h"
#include "device_common.h"
#include "launch.h"

namespace csl {

namespace {

template <int TPE, int RS, int RSX, bool HAS_Z, bool OUT_BF16, bool DUAL>
__global__ __launch_bounds__(256) void compress_kernel(
    const uint16_t* __restrict__ kv, const uint16_t* __restrict__ z, const uint16_t* __restrict__ kv_b,
    const uint16_t* __restrict__ z_b, const int64_t* __restrict__ kv_off, const int64_t* __restrict__ ent_off,
    const int64_t* __restrict__ first_entry, int D, int m, int64_t max_new, void* __restrict__ out, PagedView pg) {
  // long chunks split over waves hold 8 rows in flight per thread
  compress_block<256, TPE, RS, HAS_Z, OUT_BF16, (RSX > 1 ? 8 : 4), RSX, DUAL>(
      kv, z, kv_off, ent_off, first_entry, D, m, max_new, out, blockIdx.y, blockIdx.x, kv_b, z_b, pg);
}

struct CompressArgs {
  const void *kv, *z, *kv_b, *z_b;  // kv_b == nullptr: single series
  const int64_t *kv_off, *ent_off, *first;
  int B, D, m;
  int64_t max_new;
  void* out;
  bool out_bf16;
  PagedView pg;
};

template <int TPE, int RS, int RSX, bool DUAL>
hipError_t launch_tpe_rs(const CompressArgs& a, hipStream_t st) {
  constexpr int EPB = 256 / (TPE * RS * RSX);
  const int64_t gx = (a.max_new + EPB - 1) / EPB;
  dim3 grid((unsigned)gx, (unsigned)a.B);
  const uint16_t* k16 = static_cast<const uint16_t*>(a.kv);
  const uint16_t* z16 = static_cast<const uint16_t*>(a.z);
  const uint16_t* kb16 = static_cast<const uint16_t*>(a.kv_b);
  const uint16_t* zb16 = static_cast<const uint16_t*>(a.z_b);
#define CSL_COMPRESS_LAUNCH(HZ, OB)                                                                     \
  compress_kernel<TPE, RS, RSX, HZ, OB, DUAL><<<grid, 256, 0, st>>>(k16, z16, kb16, zb16, a.kv_off, a.ent_off, \
                                                                  a.first, a.D, a.m, a.max_new, a.out, a.pg)
  if (a.z) {
    if (a.out_bf16) CSL_COMPRESS_LAUNCH(true, true);
    else CSL_COMPRESS_LAUNCH(true, false);
  } else {
    if (a.out_bf16) CSL_COMPRESS_LAUNCH(false, true);
    else CSL_COMPRESS_LAUNCH(false, false);
  }
#undef CSL_COMPRESS_LAUNCH
  return hipGetLastError();
}

template <int TPE, bool DUAL>
hipError_t launch_tpe(const CompressArgs& a, hipStream_t st) {
  constexpr int RS_BIG = (64 / TPE) > 8 ? 8 : (64 / TPE);
  // rows pooled per entry: m, or 2m for the overlapped series
  const int rows = DUAL ? 2 * a.m : a.m;
  // Few entries (a decode step's newest chunks) of at least 8 rows per in-wave split, with a
  // full wave per entry: split the rows over up to 4 waves too, so a long chunk (m = 128)
  // loads in one round trip. Many entries (bulk compression) keep one wave per entry walking
  // its rows, which streams without workgroup turnover.
  const bool few = (int64_t)a.B * a.max_new <= 2048;
  if (few && TPE * RS_BIG == kWave && rows >= 8 * RS_BIG * 4) return launch_tpe_rs<TPE, RS_BIG, 4, DUAL>(a, st);
  if (few && TPE * RS_BIG == kWave && rows >= 8 * RS_BIG * 2) return launch_tpe_rs<TPE, RS_BIG, 2, DUAL>(a, st);
  if (rows > 8 && RS_BIG > 1) return launch_tpe_rs<TPE, RS_BIG, 1, DUAL>(a, st);
  return launch_tpe_rs<TPE, 1, 1, DUAL>(a, st);
}

template <bool DUAL>
hipError_t launch_d(const CompressArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_tpe<8, DUAL>(a, st);
    case 128: return launch_tpe<16, DUAL>(a, st);
    case 256: return launch_tpe<32, DUAL>(a, st);
    case 512: return launch_tpe<64, DUAL>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_compress(const void* kv, const void* z, const int64_t* kv_off, const int64_t* ent_off,
                           const int64_t* first_entry, int B, int D, int m, int64_t max_new_entries,
                           void* out, bool out_bf16, hipStream_t stream, const PagedView* paged) {
  const CompressArgs a{kv, z, nullptr, nullptr, kv_off, ent_off, first_entry, B, D, m, max_new_entries, out, out_bf16,
                       paged ? *paged : PagedView{}};
  return launch_d<false>(a, stream);
}

hipError_t launch_compress_overlap(const void* kv_a, const void* z_a, const void* kv_b, const void* z_b,
                                   const int64_t* kv_off, const int64_t* ent_off, const int64_t* first_entry,
                                   int B, int D, int m, int64_t max_new_entries, void* out, bool out_bf16,
                                   hipStream_t stream, const PagedView* paged) {
  const CompressArgs a{kv_a, z_a, kv_b, z_b, kv_off, ent_off, first_entry, B, D, m, max_new_entries, out, out_bf16,
                       paged ? *paged : PagedView{}};
  return launch_d<true>(a, stream);
}

}  // namespace csl

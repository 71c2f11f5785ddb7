// The attention kernels in one translation unit: the decode kernels
// (paged_decode.hip), the prefill kernels (varlen_prefill.hip), and the
// mixed-step kernel below, which runs both kinds of work in one launch.
//
// [ch15] "KV cache / batching / paged attention", section "プレフィックスキャ
// ッシュとchunked prefill": a long prefill is cut into chunks that join the
// decodes of other requests in one batch, so that the compute-heavy prefill
// and the memory-heavy decode complement each other.  [paged-doc] section
// "Varlen パス" / デコードパス: the varlen kernel can take a mixed batch, the
// decode kernel cannot.
//
// Design (gfx950): one grid.  Its first `decode_wgs` workgroups (one per CU)
// are the persistent stream-K decode workers (decode_mfma_body), the rest
// are prefill work items (prefill_body), numbered as the prefill launch
// numbers them.  Both bodies run at two waves per SIMD with at most 256
// registers a lane, so a CU can hold a decode workgroup and a prefill
// workgroup at once: the decode streams K/V from HBM while the prefill keeps
// the matrix cores busy, instead of each waiting for the other's launch.
// Which CUs receive which workgroups is the hardware dispatcher's choice
// (two decode workers may share a CU); the roles are fixed by blockIdx
// only.  The LDS of a
// workgroup is the larger of the two bodies' needs (one body runs per
// workgroup).  One-byte caches (fp8, int8) at head_dim 128: the shapes whose
// decode and prefill both run at two waves per SIMD.

#include "paged_decode.hip"
#include "varlen_prefill.hip"

namespace pkv {
namespace {

template <int CT, int D>
struct MixedLds {
  using Dl = mfd::DecodeLds<CT, D>;
  static constexpr int prefill = pf::Lds<CT, D>::bytes + 1024;  // + the flag words
  static constexpr int bytes = (Dl::bytes > prefill ? Dl::bytes : prefill);
};

template <int CT, int D, int G>
__global__ __launch_bounds__(kStreamThreads, 2) void mixed_kernel(DecodeArgs da, PrefillArgs pa, int q_tiles,
                                                                  int decode_wgs) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[MixedLds<CT, D>::bytes];
  if ((int)blockIdx.x < decode_wgs) {
    using L = mfd::DecodeLds<CT, D>;
    mfd::decode_mfma_body<CT, D, G, mfd::depth<CT>(), false>(
        da, blockIdx.x, decode_wgs, reinterpret_cast<int32_t*>(lds), reinterpret_cast<int32_t*>(lds + L::pre),
        lds + L::pre + L::part, lds + L::pre + L::part + L::chunk);
  } else {
    // one prefill work item per workgroup, numbered as the prefill launch
    // numbers them (the decode workers are a multiple of 8, so an item keeps
    // its XCD).  Taking items from the work queues instead measured no
    // faster here: the decode workers already fill the CUs' other half.
    using P = pf::Lds<CT, D>;
    pf::prefill_items<CT, D, true>(pa, q_tiles, -1, (int)blockIdx.x - decode_wgs, lds, lds + P::stage,
                                   lds + 2 * P::stage, reinterpret_cast<uint32_t*>(lds + P::bytes),
                                   reinterpret_cast<int*>(lds + P::bytes + 16));
  }
#endif
}

template <int CT, int G>
hipError_t launch_mixed_g(const DecodeArgs& da, const PrefillArgs& pa, hipStream_t stream) {
  constexpr int D = 128;
  static_assert(mfd::depth<CT>() == 2 && mfd::occupancy<CT>() == 2, "both bodies at two waves per SIMD");
  // one decode workgroup per CU (half of what the decode launch alone would
  // use: the other half of each CU runs prefill work items), never more than
  // the decode has 4-wave shares of chunks for
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int64_t max_chunks = (int64_t)da.batch * da.num_kv_heads *
                             (((int64_t)da.max_blocks_per_seq * da.block_size + kChunk - 1) / kChunk);
  int64_t dwg = (cus + 7) / 8 * 8;  // a multiple of 8, so prefill items keep their XCD numbering
  if (dwg * kWaves > max_chunks) dwg = (max_chunks + kWaves - 1) / kWaves;
  if (dwg * kWaves > kStreamMaxWaves) dwg = kStreamMaxWaves / kWaves;
  if (dwg < 1) dwg = 1;
  dwg = (dwg + 7) / 8 * 8;
  const int q_tiles = pf::tiles_of(pa.max_seqlen_q, pa.num_heads / pa.num_kv_heads, pf::col_blocks<CT, D>());
  const int64_t items = pf::grid_of(q_tiles, pa.batch, pa.num_kv_heads);
  if (items > 0x7fffffff / 2) return hipErrorInvalidValue;
  const int64_t grid = dwg + items;
  hipLaunchKernelGGL((mixed_kernel<CT, D, G>), dim3((unsigned)grid), dim3(kStreamThreads), 0, stream, da, pa,
                     q_tiles, (int)dwg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_stream_merge<kBF16, D, G>(da, 1, (int)(dwg * kWaves), stream);
}

template <int CT>
hipError_t launch_mixed_c(const DecodeArgs& da, const PrefillArgs& pa, hipStream_t stream) {
  switch (da.num_heads / da.num_kv_heads) {
    case 1: return launch_mixed_g<CT, 1>(da, pa, stream);
    case 2: return launch_mixed_g<CT, 2>(da, pa, stream);
    case 4: return launch_mixed_g<CT, 4>(da, pa, stream);
    case 8: return launch_mixed_g<CT, 8>(da, pa, stream);
    case 16: return launch_mixed_g<CT, 16>(da, pa, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_mixed(const DecodeArgs& da, const PrefillArgs& pa, hipStream_t stream) {
  if (da.head_dim != 128 || pa.head_dim != 128 || da.cache_dtype != pa.kv_dtype) return hipErrorInvalidValue;
  if (da.cache_dtype == kFP8) return launch_mixed_c<kFP8>(da, pa, stream);
  if (da.cache_dtype == kI8) return launch_mixed_c<kI8>(da, pa, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv

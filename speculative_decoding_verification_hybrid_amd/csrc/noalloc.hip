// hta_verify_attn_noalloc: the verification attention of hta_verify_attn
// without a handle and without any device allocation, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). The split-KV kernels' partial results and
// the per-sequence tree flags live in one file-scope device array, `scratch`,
// of kScratchBytes; each GPU the library runs on holds its own copy until the
// process ends. Calls on one GPU share that copy, so calls that overlap on one
// GPU (two streams, two threads) race and must be ordered by the caller.
//
// Nothing in scratch has to start at zero: every partial slot the merge reads
// and every tree flag it tests are written earlier in the same call.
#include <mutex>

#include "common.h"
#include "hta.h"
#include "hta_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;  // HTA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == (size_t)HTA_NOALLOC_SCRATCH_BYTES, "the header states the limit");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The address of this device's copy of `scratch` (the current device), looked
// up once per device. In host code the array's name is not a device address.
int scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return HTA_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return HTA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HTA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

int hta_verify_attn_noalloc(const hta_config_t* cfg, const void* q, const void* k_cache, const void* v_cache,
                            const void* k_tree, const void* v_tree, const int32_t* parent,
                            const int32_t* prefix_len, void* out, float* lse, int32_t* status, void* stream) {
  if (!q || !k_cache || !v_cache || !k_tree || !v_tree || !parent || !prefix_len || !out || !lse || !status)
    return HTA_ERR_INVALID_ARG;
  const int rc_cfg = hta_validate_config(cfg);
  if (rc_cfg != HTA_OK) return rc_cfg;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_tree) || !aligned16(v_tree) ||
      !aligned16(out))
    return HTA_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HTA_ERR_NO_DEVICE;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return HTA_ERR_NO_DEVICE;

  hta::Dims d;
  hta::PrefixLaunch pl;
  int occ = 0;
  const int rc = hta::plan_launch(cfg, cus, &d, &pl, &occ);
  if (rc != HTA_OK) return rc;

  // The same slot layout as a handle's workspace, inside scratch.
  const int64_t max_slots = (int64_t)pl.nwg + (int64_t)d.B * d.Hkv - 1;
  const bool slot_bf16 = pl.path == HTA_PATH_MFMA;
  const size_t o_bytes = align256((size_t)max_slots * d.M * d.D * (slot_bf16 ? 2 : 4));
  const size_t l_bytes = align256((size_t)max_slots * d.M * sizeof(float));
  const size_t e_bytes = align256((size_t)d.B * sizeof(int));
  if (o_bytes + l_bytes + e_bytes > kScratchBytes) return HTA_ERR_TOO_LARGE;

  void* base = nullptr;
  const int rc_s = scratch_address(dev, &base);
  if (rc_s != HTA_OK) return rc_s;
  char* b = static_cast<char*>(base);
  hta::Slots slots;
  slots.o = b;
  slots.o_bf16 = slot_bf16;
  slots.lse2 = reinterpret_cast<float*>(b + o_bytes);
  slots.o_bytes = o_bytes;
  slots.lse2_bytes = l_bytes;
  int* err_b = reinterpret_cast<int*>(b + o_bytes + l_bytes);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const hta::PrefixInputs in = {q, k_cache, v_cache, k_tree, v_tree, parent, prefix_len};
  const int rc_l = hta::launch_split(d, pl, in, slots, err_b, status, s);
  if (rc_l != HTA_OK) return rc_l;
  const int weight = pl.path == HTA_PATH_MFMA ? hta::kTreeTileWeight : 1;
  return hta::launch_merge_slots(d, pl.tile_tokens, pl.nwg, hta::tree_tiles_for(d.T, pl.tile_tokens), weight,
                                 prefix_len, slots, err_b, out, d.bf16, lse, status, s) == hipSuccess
             ? HTA_OK
             : HTA_ERR_HIP;
}

}  // extern "C"

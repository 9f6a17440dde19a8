// Library-wide entry points: version, status text, dimension checks and the
// LM-head workspace size.  Pure host code: nothing here touches the GPU.
#include "lopa_common.hpp"
#include "plan.hpp"

extern "C" int lopa_abi_version(void) { return LOPA_ABI_VERSION; }

extern "C" const char* lopa_status_string(int status) {
  switch (status) {
    case LOPA_OK: return "ok";
    case LOPA_ERR_INVALID: return "invalid argument (null pointer, size out of range or k > k_max)";
    case LOPA_ERR_UNSUPPORTED: return "valid arguments outside what the kernels support";
    case LOPA_ERR_WORKSPACE: return "workspace missing or smaller than lopa_workspace_bytes()";
    case LOPA_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case LOPA_ERR_TOO_LARGE:
      return "the call needs more than the library's fixed scratch array holds";
    default: return "unknown lopa status";
  }
}

int lopa_check_dims(const lopa_dims* d) {
  if (!d) return LOPA_ERR_INVALID;
  if (d->L < 0 || d->L > (1 << 20)) return LOPA_ERR_INVALID;
  if (d->B < 1 || d->B > LOPA_MAX_BLOCK) return LOPA_ERR_INVALID;
  if (d->Hq < 1 || d->Hkv < 1 || d->Hq % d->Hkv != 0) return LOPA_ERR_INVALID;
  if (d->d < 1 || d->d > 256) return LOPA_ERR_INVALID;
  if (d->V < 1) return LOPA_ERR_INVALID;
  if (d->k_max < 0 || d->k_max + 1 > LOPA_MAX_BRANCHES) return LOPA_ERR_INVALID;
  if (d->dtype != LOPA_F32 && d->dtype != LOPA_BF16) return LOPA_ERR_INVALID;
  const long long hidden = static_cast<long long>(d->Hq) * d->d;
  if (hidden > (1 << 16)) return LOPA_ERR_INVALID;
  // every element offset must fit in 32-bit signed arithmetic per row and the
  // whole weight in 64-bit
  if (static_cast<long long>(d->V) * hidden > (1LL << 40)) return LOPA_ERR_INVALID;
  return LOPA_OK;
}

extern "C" int lopa_workspace_bytes(const lopa_dims* dims, size_t* bytes) {
  int st = lopa_check_dims(dims);
  if (st != LOPA_OK) return st;
  if (!bytes) return LOPA_ERR_INVALID;
  *bytes = lopa::workspace_bytes(*dims);
  return LOPA_OK;
}

// C ABI of the selective-scan library: argument validation, planning and
// dispatch.  Everything up to the launch is plain host code that makes no HIP
// call, so every error path can be exercised on a machine without a GPU.
#include "../../include/ssm_scan.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "scan_internal.hpp"

namespace {

using ssm::Problem;

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const Range ra{reinterpret_cast<uintptr_t>(a), reinterpret_cast<uintptr_t>(a) + static_cast<uintptr_t>(abytes)};
  const Range rb{reinterpret_cast<uintptr_t>(b), reinterpret_cast<uintptr_t>(b) + static_cast<uintptr_t>(bbytes)};
  return ra.lo < rb.hi && rb.lo < ra.hi;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool nsplit_ok(int64_t n) { return n == 4 || n == 8 || n == 16 || n == 32 || n == 64; }

// The NSPLIT kernels address one batch row of a tensor through a buffer
// descriptor with 32-bit byte offsets: every row must stay below 2 GiB.
bool row_fits_32(const ssm_scan_args* a) {
  const int64_t lim = (int64_t{1} << 31) - 1;
  const int64_t es = a->dtype == SSM_DTYPE_F32 ? 4 : 2;
  const int64_t dmax = (a->dim > a->dstate ? a->dim : a->dstate) * es;
  return dmax > 0 && a->seqlen <= lim / dmax;
}

struct Plan {
  int variant;     // ssm_variant
  int splits;      // >= 1
  int64_t seg_len; // tokens per segment
  int64_t ws_state_bytes, ws_dsum_bytes;
};

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Element counts and the checks that need no device access.
int validate(const ssm_scan_args* a, int64_t* n_bld, int64_t* n_bln, int64_t* n_bdn) {
  if (!a) return SSM_ERR_NULL;
  if (a->batch < 0 || a->seqlen < 0 || a->dim < 0 || a->dstate < 0) return SSM_ERR_SHAPE;
  if (a->dstate < 1 || a->dstate > 64) return SSM_ERR_DSTATE;
  if (a->dtype != SSM_DTYPE_F32 && a->dtype != SSM_DTYPE_BF16) return SSM_ERR_DTYPE;
  if (a->batch > 65535) return SSM_ERR_SHAPE;  // batch rows map to grid.y
  int64_t bl, bld, bln, bd, bdn, dn;
  if (!mul_ok(a->batch, a->seqlen, &bl) || !mul_ok(bl, a->dim, &bld) || !mul_ok(bl, a->dstate, &bln) ||
      !mul_ok(a->batch, a->dim, &bd) || !mul_ok(bd, a->dstate, &bdn) || !mul_ok(a->dim, a->dstate, &dn))
    return SSM_ERR_SHAPE;
  const int64_t es = a->dtype == SSM_DTYPE_F32 ? 4 : 2;
  int64_t tmp;
  if (!mul_ok(bld, es, &tmp) || !mul_ok(bdn, 4, &tmp) || !mul_ok(bln, es, &tmp)) return SSM_ERR_SHAPE;
  if (a->flags & ~static_cast<int32_t>(SSM_FLAG_GENERIC_A)) return SSM_ERR_VARIANT;
  if (a->variant < SSM_VARIANT_AUTO || a->variant > SSM_VARIANT_DECODE) return SSM_ERR_VARIANT;
  if (a->time_splits < 0) return SSM_ERR_VARIANT;
  *n_bld = bld;
  *n_bln = bln;
  *n_bdn = bdn;
  const bool empty = bd == 0;
  if (empty) return SSM_OK;  // nothing will be read or written
  const bool has_tokens = bld > 0;
  if (has_tokens && (!a->x || !a->delta || !a->A || !a->B || !a->C || !a->y)) return SSM_ERR_NULL;
  const void* ptrs[] = {a->x, a->delta, a->A, a->B, a->C, a->D, a->z, a->delta_bias, a->h0, a->hT, a->y, a->workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSM_ERR_ALIGN;
  // Aliasing: y must not touch any input; hT may coincide with h0 exactly but
  // must not touch any other input, nor y.
  const int64_t xb = bld * es, nb = bln * es, sb = bdn * 4, db = a->dim * 4, ab = dn * 4;
  if (has_tokens) {
    const void* ins[] = {a->x, a->delta, a->B, a->C, a->z, a->A, a->D, a->delta_bias, a->h0, a->hT};
    const int64_t insz[] = {xb, xb, nb, nb, xb, ab, db, db, sb, sb};
    for (int i = 0; i < 10; ++i)
      if (overlaps(a->y, xb, ins[i], insz[i])) return SSM_ERR_ALIAS;
  }
  if (a->hT) {
    const void* ins[] = {a->x, a->delta, a->B, a->C, a->z, a->A, a->D, a->delta_bias};
    const int64_t insz[] = {xb, xb, nb, nb, xb, ab, db, db};
    for (int i = 0; i < 8; ++i)
      if (overlaps(a->hT, sb, ins[i], insz[i])) return SSM_ERR_ALIAS;
    if (a->h0 && a->h0 != a->hT && overlaps(a->hT, sb, a->h0, sb)) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

int make_plan(const ssm_scan_args* a, bool have_workspace_info, Plan* pl) {
  const int64_t N = a->dstate, L = a->seqlen;
  int variant = a->variant;
  if (variant == SSM_VARIANT_AUTO) {
    if (L == 1 && nsplit_ok(N))
      variant = SSM_VARIANT_DECODE;
    else if (nsplit_ok(N) && row_fits_32(a))
      variant = SSM_VARIANT_NSPLIT;
    else
      variant = SSM_VARIANT_LANE;
  }
  if ((variant == SSM_VARIANT_NSPLIT || variant == SSM_VARIANT_DECODE) && !nsplit_ok(N)) return SSM_ERR_VARIANT;
  if (variant == SSM_VARIANT_DECODE && L != 1) return SSM_ERR_VARIANT;
  if (variant == SSM_VARIANT_NSPLIT && !row_fits_32(a)) return SSM_ERR_VARIANT;
  if (variant != SSM_VARIANT_NSPLIT && a->time_splits > 1) return SSM_ERR_VARIANT;

  int splits = 1;
  const bool in_place = a->h0 && a->hT && a->h0 == a->hT;
  if (variant == SSM_VARIANT_NSPLIT && L > 0) {
    if (a->time_splits > 1) {
      if (in_place) return SSM_ERR_VARIANT;  // later segments read h0 after the last one wrote hT
      splits = a->time_splits;
    } else if (a->time_splits == 0 && !in_place) {
      // Split until every one of the 1024 SIMDs has a wave, keeping segments
      // at least 256 tokens long (a split costs an extra state-only pass).
      const int64_t waves = 4 * ((a->dim + 63) / 64) * a->batch;
      while (waves * splits < 1024 && L / (2 * splits) >= 256 && splits < 64) splits *= 2;
    }
  }
  int64_t seg_len = L;
  if (variant == SSM_VARIANT_NSPLIT && splits > 1) {
    seg_len = round_up((L + splits - 1) / splits, ssm::kNsplitTile);
    splits = static_cast<int>((L + seg_len - 1) / seg_len);
  }
  pl->variant = variant;
  pl->splits = splits;
  pl->seg_len = splits > 1 ? seg_len : (L > 0 ? L : 1);
  pl->ws_state_bytes = splits > 1 ? round_up(a->batch * splits * a->dim * N * 4, 256) : 0;
  pl->ws_dsum_bytes = splits > 1 ? round_up(a->batch * splits * a->dim * 4, 256) : 0;
  if (splits > 1 && have_workspace_info) {
    const int64_t need = pl->ws_state_bytes + pl->ws_dsum_bytes;
    if (!a->workspace || a->workspace_bytes < need) {
      if (a->time_splits > 1) return SSM_ERR_WORKSPACE;
      pl->splits = 1;  // automatic splitting falls back to one segment
      pl->seg_len = L;
      pl->ws_state_bytes = pl->ws_dsum_bytes = 0;
    }
  }
  return SSM_OK;
}

}  // namespace

extern "C" {

int ssm_scan_abi_version(void) { return SSM_SCAN_ABI_VERSION; }

const char* ssm_scan_strerror(int code) {
  switch (code) {
    case SSM_OK: return "success";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_SHAPE: return "invalid shape (negative extent, batch > 65535, or size overflow)";
    case SSM_ERR_DSTATE: return "dstate must be in 1..64";
    case SSM_ERR_DTYPE: return "dtype must be SSM_DTYPE_F32 or SSM_DTYPE_BF16";
    case SSM_ERR_ALIGN: return "every tensor base address must be 16-byte aligned";
    case SSM_ERR_ALIAS: return "y overlaps an input, or hT overlaps an input other than h0";
    case SSM_ERR_WORKSPACE: return "time_splits > 1 needs a workspace of ssm_scan_workspace_bytes bytes";
    case SSM_ERR_LAUNCH: return "kernel launch failed";
    case SSM_ERR_VARIANT: return "variant, flags or time_splits not valid for this problem";
    default: return "unknown status code";
  }
}

int64_t ssm_scan_workspace_bytes(const ssm_scan_args* a) {
  int64_t bld, bln, bdn;
  const int rc = validate(a, &bld, &bln, &bdn);
  if (rc != SSM_OK) return rc;
  Plan pl;
  const int prc = make_plan(a, false, &pl);
  if (prc != SSM_OK) return prc;
  return pl.ws_state_bytes + pl.ws_dsum_bytes;
}

int64_t ssm_scan_plan(const ssm_scan_args* a) {
  int64_t bld, bln, bdn;
  const int rc = validate(a, &bld, &bln, &bdn);
  if (rc != SSM_OK) return rc;
  Plan pl;
  const int prc = make_plan(a, true, &pl);
  if (prc != SSM_OK) return prc;
  return static_cast<int64_t>(pl.variant) * 65536 + pl.splits;
}

int ssm_scan_fwd(const ssm_scan_args* a, void* stream) {
  int64_t bld, bln, bdn;
  int rc = validate(a, &bld, &bln, &bdn);
  if (rc != SSM_OK) return rc;
  if (a->batch == 0 || a->dim == 0) return SSM_OK;
  Plan pl;
  rc = make_plan(a, true, &pl);
  if (rc != SSM_OK) return rc;

  Problem p;
  p.batch = a->batch;
  p.seqlen = a->seqlen;
  p.dim = a->dim;
  p.dstate = a->dstate;
  p.dtype = a->dtype;
  p.flags = a->flags;
  p.x = a->x;
  p.delta = a->delta;
  p.A = a->A;
  p.B = a->B;
  p.C = a->C;
  p.D = a->D;
  p.z = a->z;
  p.delta_bias = a->delta_bias;
  p.h0 = a->h0;
  p.hT = a->hT;
  p.y = a->y;
  p.splits = pl.splits;
  p.seg_len = pl.seg_len;
  p.ws_state = pl.splits > 1 ? static_cast<float*>(a->workspace) : nullptr;
  p.ws_dsum = pl.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(a->workspace) + pl.ws_state_bytes) : nullptr;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (a->seqlen == 0)
    e = ssm::launch_state_copy(p, s);
  else if (pl.variant == SSM_VARIANT_DECODE)
    e = ssm::launch_decode(p, s);
  else if (pl.variant == SSM_VARIANT_NSPLIT)
    e = ssm::launch_nsplit(p, s);
  else
    e = ssm::launch_lane(p, s);
  return e == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}

}  // extern "C"

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

// The NSPLIT kernels count tokens in 32 bits and address a batch row through
// buffer descriptors with 32-bit byte offsets.  A row whose accesses (up to
// 320 tokens past its end, for the prefetch) fit one 2 GiB descriptor uses
// fixed descriptors; a longer row is addressed through windows that move along
// it, with offsets under 320 tokens from the window start.  So a token of a
// row must stay below 2 GiB / 320 (D up to about 3.3 million bf16 channels);
// the row length itself is free.
int64_t nsplit_token_bytes(const ssm_scan_args* a) {
  const int64_t es = a->dtype == SSM_DTYPE_F32 ? 4 : 2;
  return (a->dim > a->dstate ? a->dim : a->dstate) * es;
}
bool nsplit_fits(const ssm_scan_args* a) {
  const int64_t lim = (int64_t{1} << 31) - 1;
  const int64_t tok = nsplit_token_bytes(a);
  return tok > 0 && tok <= lim / ssm::kNsplitReach && a->seqlen <= lim - 1024;
}
bool nsplit_windowed(const ssm_scan_args* a) {
  return (a->seqlen + ssm::kNsplitReach) * nsplit_token_bytes(a) > (int64_t{1} << 31) - 1;
}

struct Plan {
  int variant;     // ssm_variant
  int splits;      // >= 1
  int64_t seg_len; // tokens per segment
  int64_t ws_state_bytes, ws_dsum_bytes;
};

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Bytes of the forward's checkpoints for the backward: (B, ceil(L / T) - 1, 4,
// D, ceil(N / 4)) fp32 with T = ssm::ckpt_tokens(N); -1 when the count
// overflows.
int64_t ckpt_bytes(int64_t B, int64_t L, int64_t D, int64_t N) {
  const int64_t T = ssm::ckpt_tokens(N);
  const int64_t entries = L > 0 ? (L + T - 1) / T - 1 : 0;
  int64_t v;
  if (!mul_ok(B, entries, &v) || !mul_ok(v, 4 * ssm::ckpt_quarter(N), &v) || !mul_ok(v, D, &v) ||
      !mul_ok(v, 4, &v))
    return -1;
  return v;
}

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
  if (a->flags & ~static_cast<int32_t>(SSM_FLAG_GENERIC_A | SSM_FLAG_ZOH | SSM_FLAG_CARRY_SCAN)) return SSM_ERR_VARIANT;
  if (a->variant < SSM_VARIANT_AUTO || a->variant > SSM_VARIANT_DECODE) return SSM_ERR_VARIANT;
  if (a->time_splits < 0) return SSM_ERR_VARIANT;
  *n_bld = bld;
  *n_bln = bln;
  *n_bdn = bdn;
  const bool empty = bd == 0;
  if (empty) return SSM_OK;  // nothing will be read or written
  const bool has_tokens = bld > 0;
  if (has_tokens && (!a->x || !a->delta || !a->A || !a->B || !a->C || !a->y)) return SSM_ERR_NULL;
  const void* ptrs[] = {a->x, a->delta, a->A, a->B, a->C, a->D, a->z, a->delta_bias, a->h0, a->hT, a->y, a->workspace,
                        a->checkpoints};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSM_ERR_ALIGN;
  const int64_t ckb = ckpt_bytes(a->batch, a->seqlen, a->dim, a->dstate);
  if (ckb < 0) return SSM_ERR_SHAPE;
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
  if (a->checkpoints && ckb > 0) {  // an output: touches no input and no other output
    const void* others[] = {a->x, a->delta, a->B, a->C, a->z, a->A, a->D, a->delta_bias, a->h0, a->hT, a->y};
    const int64_t osz[] = {xb, xb, nb, nb, xb, ab, db, db, sb, sb, xb};
    for (int i = 0; i < 11; ++i)
      if (overlaps(a->checkpoints, ckb, others[i], osz[i])) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

int make_plan(const ssm_scan_args* a, bool have_workspace_info, Plan* pl) {
  const int64_t N = a->dstate, L = a->seqlen;
  int variant = a->variant;
  if (variant == SSM_VARIANT_AUTO) {
    if (L == 1 && nsplit_ok(N))
      variant = SSM_VARIANT_DECODE;
    else if (nsplit_ok(N) && nsplit_fits(a))
      variant = SSM_VARIANT_NSPLIT;
    else
      variant = SSM_VARIANT_LANE;
  }
  if ((variant == SSM_VARIANT_NSPLIT || variant == SSM_VARIANT_DECODE) && !nsplit_ok(N)) return SSM_ERR_VARIANT;
  if (variant == SSM_VARIANT_DECODE && L != 1) return SSM_ERR_VARIANT;
  if (variant == SSM_VARIANT_NSPLIT && !nsplit_fits(a)) return SSM_ERR_VARIANT;
  if (variant != SSM_VARIANT_NSPLIT && a->time_splits > 1) return SSM_ERR_VARIANT;

  int splits = 1;
  const bool in_place = a->h0 && a->hT && a->h0 == a->hT;
  // no chain (batch or dim 0): nothing runs, one segment and no workspace
  const bool has_chains = a->batch > 0 && a->dim > 0;
  if (variant == SSM_VARIANT_NSPLIT && L > 0 && has_chains) {
    if (a->time_splits > 1) {
      if (in_place) return SSM_ERR_VARIANT;  // later segments read h0 after the last one wrote hT
      splits = a->time_splits;
    } else if (a->time_splits == 0 && !in_place) {
      // One 8-wave block runs per compute unit at a time.  Splitting costs an
      // extra state-only pass over all but the last segment, and pays only while
      // every segment's block still finds a compute unit of its own: take the
      // most segments for which blocks x segments fits the 256 compute units,
      // keeping segments at least 256 tokens long.  (B8 L2048 D1536, 192 blocks,
      // ran 25% slower with 2 segments than with 1: the second round of blocks.
      // B1 L8192 D1536, 24 blocks: 10 segments 97 us, 8 segments 110 us, 12
      // segments 138 us.)
      constexpr int64_t kComputeUnits = 256;
      const int64_t blocks = ((a->dim + 63) / 64) * a->batch;
      int64_t fit = kComputeUnits / blocks;
      if (fit > L / 256) fit = L / 256;
      if (fit > 64) fit = 64;
      if (fit > 1) splits = static_cast<int>(fit);
    }
  }
  int64_t seg_len = L;
  if (variant == SSM_VARIANT_NSPLIT && splits > 1) {
    // an explicit split count is honoured (segments of whole tiles); automatic
    // splitting uses segments of whole half turns, which waste no padded tiles
    const int64_t unit = a->time_splits > 1 ? ssm::kNsplitTile : ssm::kNsplitTile * ssm::kNsplitTurn / 2;
    seg_len = round_up((L + splits - 1) / splits, unit);
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

// ---- backward --------------------------------------------------------------------------

struct BwdPlan {
  int splits;
  int64_t seg_len, nck, chunk;
  // byte offsets of the workspace regions, and the total
  int64_t off_ck, off_ckds, off_segh, off_segc, off_segds, off_pA, off_pD, off_pbias, off_pB, off_pC, total;
};

// Waves per batch row and segment: workgroups of G waves cover 64 channels,
// each wave 64 / G of them.  Each wave writes one partial dB / dC row.
int64_t bwd_blocks(const ssm_scan_bwd_args* a) {
  return (a->dim + 63) / 64 * ssm::bwd_lanes_per_channel(a->dstate);
}

int validate_bwd(const ssm_scan_bwd_args* a) {
  if (!a) return SSM_ERR_NULL;
  if (a->batch < 0 || a->seqlen < 0 || a->dim < 0 || a->dstate < 0) return SSM_ERR_SHAPE;
  if (a->dstate < 1 || a->dstate > ssm::kBwdMaxState) return SSM_ERR_DSTATE;
  if (a->dtype != SSM_DTYPE_F32 && a->dtype != SSM_DTYPE_BF16) return SSM_ERR_DTYPE;
  if (a->batch > 65535) return SSM_ERR_SHAPE;
  if (a->flags & ~static_cast<int32_t>(SSM_FLAG_GENERIC_A | SSM_FLAG_ZOH)) return SSM_ERR_VARIANT;
  if (a->time_splits < 0 || a->reserved != 0) return SSM_ERR_VARIANT;
  int64_t bl, bld, bln, bd, bdn, dn, tmp;
  if (!mul_ok(a->batch, a->seqlen, &bl) || !mul_ok(bl, a->dim, &bld) || !mul_ok(bl, a->dstate, &bln) ||
      !mul_ok(a->batch, a->dim, &bd) || !mul_ok(bd, a->dstate, &bdn) || !mul_ok(a->dim, a->dstate, &dn))
    return SSM_ERR_SHAPE;
  // the partial dB/dC rows hold one entry per block of 64 / G channels: B L nblk N floats
  if (!mul_ok(bln, bwd_blocks(a), &tmp) || !mul_ok(tmp, 8, &tmp) || !mul_ok(bld, 4, &tmp) ||
      !mul_ok(bdn, 4, &tmp))
    return SSM_ERR_SHAPE;
  const bool has_tokens = bld > 0;
  if (has_tokens && (!a->x || !a->delta || !a->A || !a->B || !a->C || !a->dy)) return SSM_ERR_NULL;
  if (a->dz && !a->z) return SSM_ERR_NULL;
  const void* ptrs[] = {a->x,  a->delta, a->A,  a->B,      a->C,  a->D,  a->z,           a->delta_bias,
                        a->h0, a->dy,    a->dhT, a->dx,    a->ddelta, a->dA, a->dB,      a->dC,
                        a->dD, a->dz,    a->ddelta_bias,   a->dh0, a->workspace, a->checkpoints};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSM_ERR_ALIGN;
  const int64_t ckb = ckpt_bytes(a->batch, a->seqlen, a->dim, a->dstate);
  if (ckb < 0) return SSM_ERR_SHAPE;
  const int64_t es = a->dtype == SSM_DTYPE_F32 ? 4 : 2;
  const int64_t xb = bld * es, nb = bln * es, sb = bdn * 4, db = a->dim * 4, ab = dn * 4;
  const void* ins[] = {a->x, a->delta, a->A, a->B, a->C, a->D, a->z, a->delta_bias, a->h0, a->dy, a->dhT,
                       a->checkpoints};
  const int64_t insz[] = {xb, xb, ab, nb, nb, db, xb, db, sb, xb, sb, ckb};
  const void* outs[] = {a->dx, a->ddelta, a->dA, a->dB, a->dC, a->dD, a->dz, a->ddelta_bias, a->dh0};
  const int64_t outsz[] = {xb, xb, ab, nb, nb, db, xb, db, sb};
  for (int i = 0; i < 9; ++i) {
    for (int j = 0; j < 12; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j])) return SSM_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j])) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

// Segments, chunking and workspace layout of a validated problem with B L D > 0.
int make_bwd_plan(const ssm_scan_bwd_args* a, BwdPlan* pl) {
  const int64_t L = a->seqlen, N = a->dstate;
  const int64_t T = ssm::bwd_chunk_len(N);
  const int64_t nblk = bwd_blocks(a);
  if (nblk > INT32_MAX) return SSM_ERR_SHAPE;  // blocks map to grid.x
  int64_t S = a->time_splits;
  if (S == 0) {
    // Split until there are 4096 waves (4 per SIMD), keeping segments at least
    // 64 tokens long.  The split's extra cost, an adjoint-only pass, does not
    // grow with the number of segments.
    // From the forward's checkpoints the local pass is the adjoint alone,
    // latency-bound at 84 VGPRs: it gains from more waves (measured at B4
    // L8192 D4096 on one box: 32 segments 2.523 ms, 16 segments 2.549, 8
    // segments 2.611 on another, 4 segments 2.679).
    const int64_t waves = nblk * a->batch;
    const int64_t target = a->checkpoints ? 16384 : 4096;
    S = 1;
    while (waves * S < target && L / (2 * S) >= 64 && S < 1024) S *= 2;
  }
  if (S > L) S = L;
  int64_t seg_len = round_up((L + S - 1) / S, T);
  // The kernels address a segment's tokens through buffer descriptors with
  // 32-bit byte offsets: a segment of any token tensor (and of the partial
  // dB / dC rows) must stay below 2 GiB, which may add segments.
  const int64_t es = a->dtype == SSM_DTYPE_F32 ? 4 : 2;
  int64_t per_tok = a->dim * es;
  if (nblk * N * 4 > per_tok) per_tok = nblk * N * 4;
  const int64_t max_seg = INT32_MAX / per_tok / T * T;
  if (max_seg < T) return SSM_ERR_SHAPE;
  if (seg_len > max_seg) seg_len = max_seg;
  S = (L + seg_len - 1) / seg_len;
  if (S > 65535) return SSM_ERR_VARIANT;  // segments map to grid.z
  pl->splits = static_cast<int>(S);
  pl->seg_len = seg_len;
  pl->chunk = T;
  pl->nck = (L + T - 1) / T;
  const int64_t B = a->batch, D = a->dim;
  int64_t off = 0;
  auto take = [&](int64_t floats) {
    const int64_t o = off;
    off += round_up(floats * 4, 256);
    return o;
  };
  // with the forward's checkpoints the local pass writes none of its own, and
  // the states entering segments are not combined
  const bool own_ck = a->checkpoints == nullptr;
  pl->off_ck = take(own_ck ? B * pl->nck * D * N : 0);
  pl->off_ckds = take(own_ck ? B * pl->nck * D : 0);
  pl->off_segh = take(own_ck ? B * S * D * N : 0);
  pl->off_segc = take(B * S * D * N);
  pl->off_segds = take(B * S * D);
  pl->off_pA = take(B * S * D * N);
  pl->off_pD = take(B * S * D);
  pl->off_pbias = take(B * S * D);
  pl->off_pB = take(B * L * nblk * N);  // written whether or not dB / dC are asked for
  pl->off_pC = take(B * L * nblk * N);
  pl->total = off;
  return SSM_OK;
}

bool bwd_has_work(const ssm_scan_bwd_args* a) { return a->batch > 0 && a->seqlen > 0 && a->dim > 0; }

// ---- Mamba-2 SSD ------------------------------------------------------------------------------

// Segments beyond what one grid dimension holds are not asked for.
constexpr int32_t kSsdMaxSplits = 65535;

int validate_ssd(const ssm_ssd_args* a, bool check_workspace = true) {
  if (!a) return SSM_ERR_NULL;
  if (a->batch < 0 || a->seqlen < 0 || a->nheads < 1 || a->headdim < 1 || a->ngroups < 1 || a->dstate < 1)
    return SSM_ERR_SHAPE;
  if (a->dtype != SSM_DTYPE_BF16) return a->dtype == SSM_DTYPE_F32 ? SSM_ERR_VARIANT : SSM_ERR_DTYPE;
  if (a->time_splits < 0 || a->time_splits > kSsdMaxSplits || a->headdim != 64 || a->nheads % a->ngroups != 0)
    return SSM_ERR_VARIANT;
  if (a->dstate != 64 && a->dstate != 128 && a->dstate != 256) return SSM_ERR_VARIANT;
  if (a->batch > 65535 || a->nheads > 65535) return SSM_ERR_SHAPE;
  int64_t bl, blh, xe, bn, st, tmp;
  if (!mul_ok(a->batch, a->seqlen, &bl) || !mul_ok(bl, a->nheads, &blh) || !mul_ok(blh, a->headdim, &xe) ||
      !mul_ok(bl, a->ngroups * a->dstate, &bn) || !mul_ok(a->batch * a->nheads, a->headdim * a->dstate, &st) ||
      !mul_ok(xe, 2, &tmp) || !mul_ok(st, 4, &tmp) || !mul_ok(bn, 2, &tmp))
    return SSM_ERR_SHAPE;
  const bool tokens = bl > 0;
  if (!a->A) return SSM_ERR_NULL;
  if (tokens && (!a->x || !a->dt || !a->B || !a->C || !a->y)) return SSM_ERR_NULL;
  const void* ptrs[] = {a->x, a->dt, a->A, a->B, a->C, a->D, a->dt_bias, a->h0, a->hT, a->y};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSM_ERR_ALIGN;
  const void* ins[] = {a->x, a->dt, a->A, a->B, a->C, a->D, a->dt_bias, a->h0};
  const int64_t insz[] = {xe * 2, blh * 2, a->nheads * 4, bn * 2, bn * 2, a->nheads * 4, a->nheads * 4, st * 4};
  for (int i = 0; i < 8; ++i) {
    if (overlaps(a->y, xe * 2, ins[i], insz[i])) return SSM_ERR_ALIAS;
    if (overlaps(a->hT, st * 4, ins[i], insz[i])) return SSM_ERR_ALIAS;
  }
  if (overlaps(a->hT, st * 4, a->y, xe * 2)) return SSM_ERR_ALIAS;
  if (check_workspace && a->workspace) {
    if (!aligned16(a->workspace) || a->workspace_bytes < 0) return SSM_ERR_ALIGN;
    const int64_t wb = a->workspace_bytes;
    for (int i = 0; i < 8; ++i)
      if (overlaps(a->workspace, wb, ins[i], insz[i])) return SSM_ERR_ALIAS;
    if (overlaps(a->workspace, wb, a->y, xe * 2) || overlaps(a->workspace, wb, a->hT, st * 4)) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

// Time segments of the chunked SSD / gated-attention kernel: how many, and
// the summary bytes they need.
struct SsdPlan {
  int splits = 1;
  int64_t seg_chunks = 0;
  int64_t sub_chunks = 0;  // chunks per state-only sub-segment, a divisor of seg_chunks
  int64_t ws_state = 0;    // (B, R, H, P, N) fp32, R = (S-1) seg_chunks / sub_chunks, rounded up to 256 bytes
  int64_t ws_la = 0;       // (B, R, H) fp32, rounded up to 256 bytes
  int64_t bytes() const { return ws_state + ws_la; }
};

// One workgroup runs per compute unit (its LDS use is over half of the 160 KiB),
// and one walks the chunks of one (b, h) in order.  Splitting costs a state-only
// pass over all but the last segment; it pays while every segment's workgroup
// still finds a compute unit of its own, so the automatic choice takes the most
// segments for which B H S fits the 256 compute units, with at least 4 chunks
// per segment and at most 64 segments.  Two of the state-only pass's
// workgroups fit a compute unit (its LDS would allow three, its VGPRs do not):
// each segment before the last is cut into m sub-segments, the most for which
// (S - 1) m B H fits 768 workgroups with m dividing the segment's chunks and at
// least 4 chunks each.  Past 512 they run as a second, shorter round, which
// balances the compute units better than sub-segments twice as long (B1 L32768
// H64 N128: 508 against 520 us per call).
int ssd_plan(int64_t B, int64_t L, int64_t H, int64_t N, int32_t time_splits, SsdPlan* pl) {
  constexpr int64_t kComputeUnits = 256;
  const int64_t nch = (L + 63) / 64;
  int64_t S = 1;
  if (B > 0 && nch > 0) {
    if (time_splits > 1) {
      S = time_splits;
    } else if (time_splits == 0) {
      int64_t fit = kComputeUnits / (B * H);
      if (fit > nch / 4) fit = nch / 4;
      if (fit > 64) fit = 64;
      if (fit > 1) S = fit;
    }
  }
  if (S > nch) S = nch;
  *pl = SsdPlan{};
  if (S < 2) return SSM_OK;
  const int64_t segc = (nch + S - 1) / S;
  S = (nch + segc - 1) / segc;  // no empty segment
  if (S < 2) return SSM_OK;
  int64_t m = 1;
  for (int64_t c = 2; c <= segc / 4 && c <= 3 * kComputeUnits; ++c)  // (bounds the products below)
    if (segc % c == 0 && (S - 1) * c * B * H <= 3 * kComputeUnits) m = c;
  int64_t bs, st, tmp;
  if (!mul_ok(B, (S - 1) * m, &bs) || !mul_ok(bs, H, &tmp) || !mul_ok(tmp, 64 * N * 4, &st)) return SSM_ERR_SHAPE;
  pl->splits = static_cast<int>(S);
  pl->seg_chunks = segc;
  pl->sub_chunks = segc / m;
  pl->ws_state = round_up(st, 256);
  pl->ws_la = round_up(tmp * 4, 256);
  return SSM_OK;
}

// The plan with the caller's workspace: an automatic split that does not fit
// (summaries at byte `offset` of the workspace) falls back to one segment, an
// explicit one is an error.
int ssd_plan_fit(int64_t B, int64_t L, int64_t H, int64_t N, int32_t time_splits, const void* ws, int64_t ws_bytes,
                 int64_t offset, SsdPlan* pl) {
  const int rc = ssd_plan(B, L, H, N, time_splits, pl);
  if (rc != SSM_OK) return rc;
  if (pl->splits > 1 && (!ws || ws_bytes < offset + pl->bytes())) {
    if (time_splits > 1) return SSM_ERR_WORKSPACE;
    *pl = SsdPlan{};
  }
  return SSM_OK;
}

// ---- gated linear attention / mLSTM ------------------------------------------------------

// Workspace bytes for phi(k) and phi(q): each (B, L, G, N) bf16, the second
// starting at a 256-byte boundary.
int64_t gla_ws_part(const ssm_gla_args* a) { return round_up(a->batch * a->seqlen * a->ngroups * a->dstate * 2, 256); }

int validate_gla(const ssm_gla_args* a, bool check_workspace = true) {
  if (!a) return SSM_ERR_NULL;
  if (a->batch < 0 || a->seqlen < 0 || a->nheads < 1 || a->headdim < 1 || a->ngroups < 1 || a->dstate < 1)
    return SSM_ERR_SHAPE;
  if (a->dtype != SSM_DTYPE_BF16) return a->dtype == SSM_DTYPE_F32 ? SSM_ERR_VARIANT : SSM_ERR_DTYPE;
  if (a->feature_map < 0 || a->feature_map > 1 || a->headdim != 64 || a->nheads % a->ngroups != 0 ||
      a->reserved != 0 || a->time_splits < 0 || a->time_splits > kSsdMaxSplits)
    return SSM_ERR_VARIANT;
  if (a->dstate != 64 && a->dstate != 128 && a->dstate != 256) return SSM_ERR_VARIANT;
  if (a->batch > 65535 || a->nheads > 65535) return SSM_ERR_SHAPE;
  int64_t bl, blh, ve, qk, st, tmp;
  if (!mul_ok(a->batch, a->seqlen, &bl) || !mul_ok(bl, a->nheads, &blh) || !mul_ok(blh, a->headdim, &ve) ||
      !mul_ok(bl, a->ngroups * a->dstate, &qk) || !mul_ok(a->batch * a->nheads, a->headdim * a->dstate, &st) ||
      !mul_ok(ve, 2, &tmp) || !mul_ok(st, 4, &tmp) || !mul_ok(qk, 2, &tmp) || !mul_ok(blh, 4, &tmp))
    return SSM_ERR_SHAPE;
  if (bl > 0 && (!a->q || !a->k || !a->v || !a->y)) return SSM_ERR_NULL;
  const void* ptrs[] = {a->q, a->k, a->v, a->log_f, a->in_gate, a->h0, a->hT, a->y};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSM_ERR_ALIGN;
  const void* ins[] = {a->q, a->k, a->v, a->log_f, a->in_gate, a->h0};
  const int64_t insz[] = {qk * 2, qk * 2, ve * 2, blh * 4, blh * 4, st * 4};
  for (int i = 0; i < 6; ++i) {
    if (overlaps(a->y, ve * 2, ins[i], insz[i])) return SSM_ERR_ALIAS;
    if (overlaps(a->hT, st * 4, ins[i], insz[i])) return SSM_ERR_ALIAS;
  }
  if (overlaps(a->hT, st * 4, a->y, ve * 2)) return SSM_ERR_ALIAS;
  if (check_workspace && a->workspace) {
    if (!aligned16(a->workspace) || a->workspace_bytes < 0) return SSM_ERR_ALIGN;
    const int64_t wb = a->workspace_bytes;
    for (int i = 0; i < 6; ++i)
      if (overlaps(a->workspace, wb, ins[i], insz[i])) return SSM_ERR_ALIAS;
    if (overlaps(a->workspace, wb, a->y, ve * 2) || overlaps(a->workspace, wb, a->hT, st * 4)) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

// ---- conv1d + SiLU prologue ---------------------------------------------------------------

int validate_conv(const ssm_conv_args* a) {
  if (!a) return SSM_ERR_NULL;
  if (a->batch < 0 || a->seqlen < 0 || a->dim < 0) return SSM_ERR_SHAPE;
  if (a->dtype != SSM_DTYPE_F32 && a->dtype != SSM_DTYPE_BF16) return SSM_ERR_DTYPE;
  if (a->width < 1 || a->width > 4) return SSM_ERR_VARIANT;
  if (a->batch > 65535) return SSM_ERR_SHAPE;  // batch rows map to grid.z
  const int64_t H = a->width - 1;
  int64_t bl, bld, bhd, dw, tmp;
  if (!mul_ok(a->batch, a->seqlen, &bl) || !mul_ok(bl, a->dim, &bld) || !mul_ok(a->batch * H, a->dim, &bhd) ||
      !mul_ok(a->dim, a->width, &dw) || !mul_ok(bld, 4, &tmp) || !mul_ok(bhd, 4, &tmp) || !mul_ok(dw, 4, &tmp))
    return SSM_ERR_SHAPE;
  if (bld > 0 && (!a->x || !a->weight || !a->u)) return SSM_ERR_NULL;
  const void* ptrs[] = {a->x, a->weight, a->bias, a->state, a->u, a->state_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSM_ERR_ALIGN;
  const int64_t es = a->dtype == SSM_DTYPE_F32 ? 4 : 2;
  const int64_t xb = bld * es, sb = bhd * es;
  const void* ins[] = {a->x, a->weight, a->bias, a->state};
  const int64_t insz[] = {xb, dw * 4, a->dim * 4, sb};
  for (int i = 0; i < 4; ++i) {
    if (overlaps(a->u, xb, ins[i], insz[i])) return SSM_ERR_ALIAS;
    if (overlaps(a->state_out, sb, ins[i], insz[i])) return SSM_ERR_ALIAS;
  }
  if (overlaps(a->state_out, sb, a->u, xb)) return SSM_ERR_ALIAS;
  return SSM_OK;
}

}  // namespace

extern "C" {

int ssm_scan_abi_version(void) { return SSM_SCAN_ABI_VERSION; }

const char* ssm_scan_strerror(int code) {
  switch (code) {
    case SSM_OK: return "success";
    case SSM_ERR_NULL: return "a required pointer is NULL (or dz given without z)";
    case SSM_ERR_SHAPE: return "invalid shape (negative extent, batch > 65535, or size overflow)";
    case SSM_ERR_DSTATE: return "dstate out of range (1..64)";
    case SSM_ERR_DTYPE: return "dtype must be SSM_DTYPE_F32 or SSM_DTYPE_BF16";
    case SSM_ERR_ALIGN: return "every tensor base address must be 16-byte aligned";
    case SSM_ERR_ALIAS: return "an output overlaps an input or another output (hT may equal h0)";
    case SSM_ERR_WORKSPACE: return "workspace missing or smaller than the *_workspace_bytes query returns";
    case SSM_ERR_LAUNCH: return "kernel launch failed";
    case SSM_ERR_VARIANT: return "variant, flags, time_splits or reserved not valid for this problem";
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

namespace {

// Launch a validated, planned forward call; ws is the segment summaries'
// memory when the plan splits time.
int run_fwd(const ssm_scan_args* a, const Plan& pl, void* ws, void* stream) {
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
  p.windowed = pl.variant == SSM_VARIANT_NSPLIT && nsplit_windowed(a);
  p.ws_state = pl.splits > 1 ? static_cast<float*>(ws) : nullptr;
  p.ws_dsum = pl.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + pl.ws_state_bytes) : nullptr;
  p.checkpoints = ckpt_bytes(a->batch, a->seqlen, a->dim, a->dstate) > 0 ? a->checkpoints : nullptr;

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

}  // namespace

int64_t ssm_scan_checkpoint_bytes(const ssm_scan_args* a) {
  int64_t bld, bln, bdn;
  const int rc = validate(a, &bld, &bln, &bdn);
  if (rc != SSM_OK) return rc;
  return ckpt_bytes(a->batch, a->seqlen, a->dim, a->dstate);
}

int ssm_scan_fwd(const ssm_scan_args* a, void* stream) {
  int64_t bld, bln, bdn;
  int rc = validate(a, &bld, &bln, &bdn);
  if (rc != SSM_OK) return rc;
  if (a->batch == 0 || a->dim == 0) return SSM_OK;
  Plan pl;
  rc = make_plan(a, true, &pl);
  if (rc != SSM_OK) return rc;
  return run_fwd(a, pl, a->workspace, stream);
}

int ssm_scan_fwd_noalloc(const ssm_scan_args* a, void* stream) {
  int64_t bld, bln, bdn;
  int rc = validate(a, &bld, &bln, &bdn);
  if (rc != SSM_OK) return rc;
  if (a->batch == 0 || a->dim == 0) return SSM_OK;
  // the plan as if a workspace of any size were given; the caller's own
  // workspace fields play no part
  ssm_scan_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  Plan pl;
  rc = make_plan(&b, false, &pl);
  if (rc != SSM_OK) return rc;
  void* ws = nullptr;
  if (pl.splits > 1) {
    if (pl.ws_state_bytes + pl.ws_dsum_bytes > ssm::kNoallocScratchBytes) {
      if (a->time_splits > 1) return SSM_ERR_WORKSPACE;
      pl.splits = 1;  // automatic splitting falls back to one segment
      pl.seg_len = a->seqlen;
      pl.ws_state_bytes = pl.ws_dsum_bytes = 0;
    } else if (ssm::noalloc_scratch(&ws) != hipSuccess) {
      return SSM_ERR_LAUNCH;
    }
  }
  return run_fwd(&b, pl, ws, stream);
}

int64_t ssm_scan_bwd_workspace_bytes(const ssm_scan_bwd_args* a) {
  const int rc = validate_bwd(a);
  if (rc != SSM_OK) return rc;
  if (!bwd_has_work(a)) return 0;
  BwdPlan pl;
  const int prc = make_bwd_plan(a, &pl);
  return prc != SSM_OK ? prc : pl.total;
}

int64_t ssm_scan_bwd_plan(const ssm_scan_bwd_args* a) {
  const int rc = validate_bwd(a);
  if (rc != SSM_OK) return rc;
  if (!bwd_has_work(a)) return 1;
  BwdPlan pl;
  const int prc = make_bwd_plan(a, &pl);
  return prc != SSM_OK ? prc : pl.splits;
}

int ssm_scan_bwd(const ssm_scan_bwd_args* a, void* stream) {
  int rc = validate_bwd(a);
  if (rc != SSM_OK) return rc;
  ssm::BwdProblem p{};
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
  p.dy = a->dy;
  p.dhT = a->dhT;
  p.dx = a->dx;
  p.ddelta = a->ddelta;
  p.dA = a->dA;
  p.dB = a->dB;
  p.dC = a->dC;
  p.dD = a->dD;
  p.dz = a->dz;
  p.ddelta_bias = a->ddelta_bias;
  p.dh0 = a->dh0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (!bwd_has_work(a)) {
    e = ssm::launch_bwd_empty(p, s);
    return e == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
  }
  BwdPlan pl;
  rc = make_bwd_plan(a, &pl);
  if (rc != SSM_OK) return rc;
  if (!a->workspace || a->workspace_bytes < pl.total) return SSM_ERR_WORKSPACE;
  char* w = static_cast<char*>(a->workspace);
  auto reg = [&](int64_t off) { return reinterpret_cast<float*>(w + off); };
  p.splits = pl.splits;
  p.seg_len = pl.seg_len;
  p.nck = pl.nck;
  p.nblk = bwd_blocks(a);
  p.ck = reg(pl.off_ck);
  p.ckds = reg(pl.off_ckds);
  p.segh = reg(pl.off_segh);
  p.segc = reg(pl.off_segc);
  p.segds = reg(pl.off_segds);
  p.pA = reg(pl.off_pA);
  p.pD = reg(pl.off_pD);
  p.pbias = reg(pl.off_pbias);
  p.pB = reg(pl.off_pB);
  p.pC = reg(pl.off_pC);
  p.ck_in = a->checkpoints;
  e = ssm::launch_bwd(p, s);
  return e == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}

int ssm_conv1d_silu_fwd(const ssm_conv_args* a, void* stream) {
  const int rc = validate_conv(a);
  if (rc != SSM_OK) return rc;
  if (a->batch == 0 || a->dim == 0) return SSM_OK;
  ssm::ConvProblem p;
  p.batch = a->batch;
  p.seqlen = a->seqlen;
  p.dim = a->dim;
  p.width = a->width;
  p.dtype = a->dtype;
  p.x = a->x;
  p.weight = a->weight;
  p.bias = a->bias;
  p.state = a->state;
  p.u = a->u;
  p.state_out = a->state_out;
  const hipError_t e = ssm::launch_conv(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}

namespace {

// Segment fields of a kernel problem from a plan; summaries at `ws`.
void set_segments(ssm::SsdProblem* p, const SsdPlan& pl, void* ws) {
  p->splits = pl.splits;
  p->seg_chunks = pl.seg_chunks;
  p->sub_chunks = pl.sub_chunks;
  if (pl.splits > 1) {
    p->ws_state = static_cast<float*>(ws);
    p->ws_la = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.ws_state);
  }
}

}  // namespace

int ssm_ssd_fwd(const ssm_ssd_args* a, void* stream) {
  const int rc = validate_ssd(a);
  if (rc != SSM_OK) return rc;
  if (a->batch == 0) return SSM_OK;
  ssm::SsdProblem p;
  p.batch = a->batch;
  p.seqlen = a->seqlen;
  p.nheads = a->nheads;
  p.headdim = a->headdim;
  p.ngroups = a->ngroups;
  p.dstate = a->dstate;
  p.x = a->x;
  p.dt = a->dt;
  p.A = a->A;
  p.B = a->B;
  p.C = a->C;
  p.D = a->D;
  p.dt_bias = a->dt_bias;
  p.h0 = a->h0;
  p.hT = a->hT;
  p.y = a->y;
  SsdPlan pl;
  const int prc = ssd_plan_fit(a->batch, a->seqlen, a->nheads, a->dstate, a->time_splits, a->workspace,
                               a->workspace_bytes, 0, &pl);
  if (prc != SSM_OK) return prc;
  set_segments(&p, pl, a->workspace);
  const hipError_t e = ssm::launch_ssd(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}

int64_t ssm_ssd_workspace_bytes(const ssm_ssd_args* a) {
  const int rc = validate_ssd(a, false);
  if (rc != SSM_OK) return rc;
  SsdPlan pl;
  const int prc = ssd_plan(a->batch, a->seqlen, a->nheads, a->dstate, a->time_splits, &pl);
  return prc != SSM_OK ? prc : pl.bytes();
}

int ssm_ssd_plan(const ssm_ssd_args* a) {
  const int rc = validate_ssd(a);
  if (rc != SSM_OK) return rc;
  SsdPlan pl;
  const int prc = ssd_plan_fit(a->batch, a->seqlen, a->nheads, a->dstate, a->time_splits, a->workspace,
                               a->workspace_bytes, 0, &pl);
  return prc != SSM_OK ? prc : pl.splits;
}

namespace {

// Bytes in front of the segment summaries in a gated-attention workspace:
// phi(k) and phi(q) with the feature map.
int64_t gla_phi_bytes(const ssm_gla_args* a) {
  return a->feature_map == 1 && a->batch > 0 && a->seqlen > 0 ? 2 * gla_ws_part(a) : 0;
}

}  // namespace

int ssm_gla_fwd(const ssm_gla_args* a, void* stream) {
  const int rc = validate_gla(a);
  if (rc != SSM_OK) return rc;
  if (a->batch == 0) return SSM_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  SsdPlan pl;
  const int64_t phi = gla_phi_bytes(a);
  const int prc = ssd_plan_fit(a->batch, a->seqlen, a->nheads, a->dstate, a->time_splits, a->workspace,
                               a->workspace_bytes, phi, &pl);
  if (prc != SSM_OK) return prc;
  // feature map applied once per call into the workspace when one is given
  const int64_t part = gla_ws_part(a);
  const bool prepass = phi > 0 && a->workspace && a->workspace_bytes >= phi;
  const void* keys = a->k;
  const void* queries = a->q;
  if (prepass) {
    void* pk = a->workspace;
    void* pq = static_cast<char*>(a->workspace) + part;
    const int64_t n = a->batch * a->seqlen * a->ngroups * a->dstate;
    const hipError_t fe = ssm::launch_gla_feature_map(a->k, a->q, pk, pq, n, s);
    if (fe != hipSuccess) return SSM_ERR_LAUNCH;
    keys = pk;
    queries = pq;
  }
  ssm::SsdProblem p;
  p.batch = a->batch;
  p.seqlen = a->seqlen;
  p.nheads = a->nheads;
  p.headdim = a->headdim;
  p.ngroups = a->ngroups;
  p.dstate = a->dstate;
  p.mode = prepass ? 1 : 1 + a->feature_map;
  p.x = a->v;  // values play the role of x, keys of B, queries of C
  p.dt = nullptr;
  p.A = nullptr;
  p.B = keys;
  p.C = queries;
  p.D = nullptr;
  p.dt_bias = nullptr;
  p.log_f = a->log_f;
  p.in_gate = a->in_gate;
  p.h0 = a->h0;
  p.hT = a->hT;
  p.y = a->y;
  set_segments(&p, pl, pl.splits > 1 ? static_cast<char*>(a->workspace) + phi : nullptr);
  const hipError_t e = ssm::launch_ssd(p, s);
  return e == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}

int64_t ssm_gla_workspace_bytes(const ssm_gla_args* a) {
  const int rc = validate_gla(a, false);
  if (rc != SSM_OK) return rc;
  SsdPlan pl;
  const int prc = ssd_plan(a->batch, a->seqlen, a->nheads, a->dstate, a->time_splits, &pl);
  return prc != SSM_OK ? prc : gla_phi_bytes(a) + pl.bytes();
}

int ssm_gla_plan(const ssm_gla_args* a) {
  const int rc = validate_gla(a);
  if (rc != SSM_OK) return rc;
  SsdPlan pl;
  const int prc = ssd_plan_fit(a->batch, a->seqlen, a->nheads, a->dstate, a->time_splits, a->workspace,
                               a->workspace_bytes, gla_phi_bytes(a), &pl);
  return prc != SSM_OK ? prc : pl.splits;
}

}  // extern "C"

// fp8 (OCP E4M3 Q/K with per-token scales, bf16 V) instantiations of the
// matrix-core attention kernel: D 128, and D 128 with a bfloat16 rope part
// of 64 (the scales then cover the nope product only).
#include "attn_mfma.h"

namespace mha {
namespace {
using C128 = MfmaCfg<128, 0, 128, true>;
using CRope = MfmaCfg<128, 64, 128, true>;
const Variant kFp8[] = {
    {launch_mfma<C128>, blocks_mfma<C128>, C128::BM, C128::BN, C128::LDS, launch_mfma<C128, true>},
    {launch_mfma<CRope>, blocks_mfma<CRope>, CRope::BM, CRope::BN, CRope::LDS,
     launch_mfma<CRope, true>},
};
}  // namespace

const Variant* find_variant_fp8(int dn, int dr, int dv) {
  if (dn == 128 && dr == 0 && dv == 128) return &kFp8[0];
  if (dn == 128 && dr == 64 && dv == 128) return &kFp8[1];
  return nullptr;
}
}  // namespace mha

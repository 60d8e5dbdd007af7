// fp8 (OCP E4M3 Q/K with per-token scales, bf16 V) instantiations of the
// matrix-core attention kernel: D 128, and D 128 with a bfloat16 rope part
// of 64 (the scales then cover the nope product only).  Two sets: the codes
// decoded to bfloat16 for the Q K^T products (exact products, float32-grade
// accumulation), and the products on the fp8 matrix instruction (twice the
// rate, accumulation limited to about 13 bits below the largest product).
#include "attn_mfma.h"

namespace mha {
namespace {
using C128 = MfmaCfg<128, 0, 128, true, false>;
using CRope = MfmaCfg<128, 64, 128, true, false>;
using F128 = MfmaCfg<128, 0, 128, true, true>;
using FRope = MfmaCfg<128, 64, 128, true, true>;
const Variant kFp8[] = {
    {launch_mfma<C128>, blocks_mfma<C128>, C128::BM, C128::BN, C128::LDS, launch_mfma<C128, true>},
    {launch_mfma<CRope>, blocks_mfma<CRope>, CRope::BM, CRope::BN, CRope::LDS,
     launch_mfma<CRope, true>},
};
const Variant kFp8Fast[] = {
    {launch_mfma<F128>, blocks_mfma<F128>, F128::BM, F128::BN, F128::LDS, launch_mfma<F128, true>},
    {launch_mfma<FRope>, blocks_mfma<FRope>, FRope::BM, FRope::BN, FRope::LDS,
     launch_mfma<FRope, true>},
};
}  // namespace

const Variant* find_variant_fp8(int dn, int dr, int dv, bool fast) {
  const Variant* v = fast ? kFp8Fast : kFp8;
  if (dn == 128 && dr == 0 && dv == 128) return &v[0];
  if (dn == 128 && dr == 64 && dv == 128) return &v[1];
  return nullptr;
}
}  // namespace mha

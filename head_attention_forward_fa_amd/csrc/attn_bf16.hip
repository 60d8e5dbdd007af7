// bf16 instantiations of the matrix-core attention kernel.
#include "attn_mfma.h"

namespace mha {
namespace {
using C64 = MfmaCfg<64, 0, 64, false>;
using C128 = MfmaCfg<128, 0, 128, false>;
using CRope = MfmaCfg<128, 64, 128, false>;
const Variant kBf16[] = {
    {launch_mfma<C64>, blocks_mfma<C64>, C64::BM, C64::BN, C64::LDS, launch_mfma<C64, true>},
    {launch_mfma<C128>, blocks_mfma<C128>, C128::BM, C128::BN, C128::LDS, launch_mfma<C128, true>},
    {launch_mfma<CRope>, blocks_mfma<CRope>, CRope::BM, CRope::BN, CRope::LDS, launch_mfma<CRope, true>},
};
}  // namespace

const Variant* find_variant_bf16(int dn, int dr, int dv) {
  if (dn == 64 && dr == 0 && dv == 64) return &kBf16[0];
  if (dn == 128 && dr == 0 && dv == 128) return &kBf16[1];
  if (dn == 128 && dr == 64 && dv == 128) return &kBf16[2];
  return nullptr;
}
}  // namespace mha

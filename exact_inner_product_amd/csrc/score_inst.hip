// score_inst.hip -- instantiates the score pass for one corpus dtype and width, given as
// MIPS_CT (MIPS_F32, MIPS_BF16, MIPS_FP8_E4M3 or MIPS_INT8) and MIPS_D by the build; one object per
// pair keeps each compilation small and lets them run in parallel.
#include "score.h"

#if !defined(MIPS_CT) || !defined(MIPS_D)
#error "MIPS_CT and MIPS_D must be defined"
#endif

namespace mips {
template int launch_score_nqf<MIPS_CT, MIPS_D, MODE_MAIN>(int, const ScoreArgs&, int, hipStream_t, hipEvent_t,
                                                                   hipEvent_t);
template int launch_score_nqf<MIPS_CT, MIPS_D, MODE_SAMPLE>(int, const ScoreArgs&, int, hipStream_t, hipEvent_t,
                                                                   hipEvent_t);
template int launch_score_nqf<MIPS_CT, MIPS_D, MODE_DENSE>(int, const ScoreArgs&, int, hipStream_t, hipEvent_t,
                                                                   hipEvent_t);
// multi-mask passes
template int launch_score_nqf<MIPS_CT, MIPS_D, MODE_MAIN, kMaxMasks>(int, const ScoreArgs&, int, hipStream_t, hipEvent_t,
                                                                   hipEvent_t);
template int launch_score_nqf<MIPS_CT, MIPS_D, MODE_SAMPLE, kMaxMasks>(int, const ScoreArgs&, int, hipStream_t, hipEvent_t,
                                                                   hipEvent_t);
template int launch_score_nqf<MIPS_CT, MIPS_D, MODE_DENSE, kMaxMasks>(int, const ScoreArgs&, int, hipStream_t, hipEvent_t,
                                                                   hipEvent_t);
}  // namespace mips

// Constants of the RoPE table's exact evaluation (k_rope.hip), kept in a header of their
// own so that the host test shim can hand them to the CPU tests, which check every digit
// against arbitrary-precision values.
#pragma once

// The first 320 bits of 2/pi, 32 to a word, most significant first: the argument
// reduction multiplies an f32 angle by a window of these bits.
#define KVC_TWO_OVER_PI_WORDS                                                                 \
    0xa2f9836eu, 0x4e441529u, 0xfc2757d1u, 0xf534ddc0u, 0xdb629599u, 0x3c439041u, 0xfe5163abu, \
        0xdebbc561u, 0xb7246e3au, 0x424dd2e0u
#define KVC_TWO_OVER_PI_NWORDS 10

// pi/2 and ln 2 as unevaluated sums hi + lo of two doubles (hi the nearest double, lo the
// nearest double to the rest).
#define KVC_PI_2_HI 0x1.921fb54442d18p+0
#define KVC_PI_2_LO 0x1.1a62633145c07p-54
#define KVC_LN2_HI 0x1.62e42fefa39efp-1
#define KVC_LN2_LO 0x1.abc9e3b39803fp-56

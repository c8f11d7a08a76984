// Host stand-in for the HIP device environment, so that a kernel source can
// be compiled for the CPU and run with one host thread per GPU lane (see
// emu.h).  Only what the indexer-logits source and the shared device header
// use is provided; device builtins that source does not call abort if
// reached.
#pragma once
#include "hip_runtime_api.h"
#include "../emu.h"

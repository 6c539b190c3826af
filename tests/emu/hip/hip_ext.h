// Test infrastructure: hipExtLaunchKernelGGL of the CPU stand-in (events ignored).
#pragma once
#include <hip/hip_runtime.h>
#define hipExtLaunchKernelGGL(K, G, B, SH, ST, E0, E1, FL, ...) emu_launch(#K, K, G, B, __VA_ARGS__)

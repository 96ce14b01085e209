// Launch bookkeeping of the host-only HIP stand-in (fake_hip.cpp).
#pragma once
#ifdef __cplusplus
extern "C" {
#endif
long fake_hip_launches(void);       // kernel launches so far
long fake_hip_bad_launches(void);   // launches outside the gfx950 limits
const char* fake_hip_last_kernel(void);
unsigned fake_hip_last_grid_x(void);   // grid and block of the last launch
unsigned fake_hip_last_block_x(void);
#ifdef __cplusplus
}
#endif

"""MI355X-native persistent decode megakernel: ctypes binding (mk) over
libmk.so and torch plumbing (engine).  Importing the package does not load
the library; the first call does, and fails loudly if it is not built."""
